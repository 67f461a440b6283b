"""Pins that tie the CPU oracle to the pages and to mathematics other than itself.

Each pin is a plain function taking an oracle instance and raising AssertionError on a
mismatch; test_oracle_pins.py runs them on the real oracle and test_oracle_mutants.py runs
them on deliberately broken copies of it (every mutant must fail at least one pin).

Pages (cited by title and section):
  DataCamp "MatMul-free language models": "Replacing MatMul with ternary operations",
  "Core components: MLGRU and GLU".  Hysen Labs "MatMul-Free LM": "FusedBitLinear",
  "HGRN attention: gated recurrence replaces softmax".
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _bf(x):
    """Exact bf16 rounding of fp32 values (test-side, for building inputs)."""
    from ternary_weight_matmul_bitlinear_amd.synth import round_to_bf16
    return round_to_bf16(np.asarray(x, np.float32))


# --------------------------------------------------------------------- quantizers

def pin_act_quant_hand(orc):
    """HC1-HC5 and the all-zero row: hand-derived int8 codes (ties to even)."""
    g = _golden("act_quant_hand.json")
    for case in g["cases"]:
        x = np.array([case["x"]], np.float32)
        q, a, rs = orc.act_quant(x)
        assert q[0].tolist() == case["q"], (case["id"], q[0].tolist(), case["q"])
        assert rs[0] == sum(case["q"]), case["id"]
    # dequantization scale of HC4: a = r * max|x| / 127 with r = 1/sqrt(mean x^2 + eps)
    x = np.array([[254, 5, -127, 0]], np.float32)
    _, a, _ = orc.act_quant(x, eps=1e-6)
    expect = 254.0 / 127.0 / math.sqrt((254**2 + 25 + 127**2) / 4 + 1e-6)
    assert abs(a[0] - expect) <= 1e-15 * expect, (a[0], expect)
    # all-zero row: the floored max (fp32 1e-5) gives a = 1e-5 / 127 / sqrt(eps)
    _, a, _ = orc.act_quant(np.zeros((1, 4), np.float32), eps=1e-6)
    expect = float(np.float32(1e-5)) / 127.0 / math.sqrt(1e-6)
    assert abs(a[0] - expect) <= 1e-15 * expect, (a[0], expect)


def pin_ternarize_hand(orc):
    """HC6: absmean scale 0.5; -0.5 ties round to 0.  HCfloor0/1: an all-zero and an
    all-tiny matrix take the floored scale fp32(1e-5), so every code is 0."""
    g = _golden("ternarize_hand.json")
    for case in g["cases"]:
        q, s = orc.ternarize(np.array(case["w"], np.float32))
        assert q.tolist() == case["q"], (case["id"], q.tolist())
        assert s == case.get("s", case["mean_abs"]), (case["id"], s)


def pin_pack_format(orc):
    """The documented 2-bit layout: code = q + 1, element 16j + 4a + b at bits 8b + 2a."""
    g = _golden("pack_format.json")
    q = np.array([g["q"]], np.int8)
    p = orc.pack(q)
    assert int(p[0, 0]) == int(g["word"], 16), hex(int(p[0, 0]))
    assert orc.unpack(p, 16).tolist() == [g["q"]]
    bad = np.array([[int(g["invalid_word"], 16)]], np.uint32)
    try:
        orc.unpack(bad, 16)
    except ValueError:
        pass
    else:
        raise AssertionError("code 3 accepted")


def pin_trit_pack_hand(orc):
    """Base-3 packing, five trits per byte: hand-worked bytes from the definition
    b = ceil(256 v / 243), v = sum_i c_i 3^(4-i); the strided byte layout of a 20-trit word;
    padding with code 1; the inverse v = floor(243 b / 256); a byte no group packs to."""
    g = _golden("trit_pack_hand.json")
    for case in g["bytes"]:
        c = case["codes"]
        # a 20-trit row whose byte 0 holds these codes and whose other bytes are all zeros (q = 0)
        q = np.zeros((1, 20), np.int8)
        for i, ci in enumerate(c):
            q[0, 4 * i] = ci - 1
        p = orc.pack_trits(q)
        assert int(p[0, 0]) == case["b"], (c, int(p[0, 0]))
        assert np.all(p[0, 1:] == 128)
        assert np.array_equal(orc.unpack_trits(p, 20), q)
    r = g["row20"]
    q = np.array([r["q"]], np.int8)
    p = orc.pack_trits(q)
    assert p[0].tolist() == r["packed"], p[0].tolist()
    assert np.array_equal(orc.unpack_trits(p, 20), q)
    r = g["row64_plus_one"]
    p = orc.pack_trits(np.full((1, r["k"]), r["q_value"], np.int8))
    assert p[0].tolist() == r["packed"], p[0].tolist()
    inv = g["inverse"]
    row = np.full((1, 16), 128, np.uint8)
    row[0, 0] = inv["b"]
    qq = orc.unpack_trits(row, 20)
    assert [int(qq[0, 4 * i]) + 1 for i in range(5)] == inv["codes"]
    for bad in (g["invalid_byte"]["b"],):
        row[0, 0] = bad
        try:
            orc.unpack_trits(row, 20)
        except ValueError:
            pass
        else:
            raise AssertionError(f"byte {bad} accepted")
    row[0, 0] = 128
    row64 = np.array([r["packed"]], np.uint8)
    row64[0, 12] = 255                       # padding digits 1..4 of word 3 set to code 2
    try:
        orc.unpack_trits(row64, 64)
    except ValueError:
        pass
    else:
        raise AssertionError("non-zero padding accepted")


def pin_trit_invariants(orc):
    """Round trip on random ternary rows of several lengths; the trit and 2-bit formats
    decode to the same weights; only 243 byte values ever occur; a row costs 16 bytes per
    80 weights (1.6 bits each)."""
    rng = np.random.default_rng(21)
    seen = set()
    for k in (64, 80, 1024, 2048, 2816):
        q = rng.integers(-1, 2, (33, k)).astype(np.int8)
        p = orc.pack_trits(q)
        assert p.shape == (33, 16 * ((k + 79) // 80))
        assert np.array_equal(orc.unpack_trits(p, k), q)
        assert np.array_equal(orc.unpack_trits(p, k), orc.unpack(orc.pack(q), k))
        seen |= set(np.unique(p).tolist())
    assert len(seen) <= 243 and 1 not in seen
    assert orc.trit_row_bytes(2048) == 416 and orc.trit_row_bytes(80) == 16


def pin_quant_invariants(orc):
    """q in [-127,127]; every non-zero row reaches +-127 at its max; sign kept; monotone;
    scaling the row by 2^k leaves q unchanged; rowsum is the sum of q."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 1024)).astype(np.float32) * np.float32(3.0)
    x[5] = 0.0
    q, a, rs = orc.act_quant(x)
    assert q.min() >= -127 and q.max() <= 127
    for r in range(64):
        if r == 5:
            assert not q[r].any()
            continue
        j = int(np.argmax(np.abs(x[r])))
        assert abs(int(q[r, j])) == 127
        assert np.all((np.sign(q[r]) == np.sign(x[r])) | (q[r] == 0))
        order = np.argsort(x[r], kind="stable")
        assert np.all(np.diff(q[r][order].astype(np.int32)) >= 0)
    assert np.array_equal(rs, q.astype(np.int32).sum(axis=1))
    for k in (-7, 3, 20):
        q2, _, _ = orc.act_quant(x * np.float32(2.0**k))
        assert np.array_equal(q, q2), k


def pin_quant_literal_rmsnorm(orc):
    """fp64 literal 'RMSNorm, then absmax-quantize' agrees with the canonical form except
    by +-1 at elements within rounding distance of a .5 tie; the gain is applied."""
    rng = np.random.default_rng(12)
    x = _bf(rng.standard_normal((256, 2048)))
    gamma = (1.0 + 0.25 * rng.standard_normal(2048)).astype(np.float32)
    q, a, _ = orc.act_quant(x, gamma=gamma, eps=1e-6)
    xd = x.astype(np.float64)
    r = 1.0 / np.sqrt((xd * xd).mean(axis=1, keepdims=True) + 1e-6)
    y = xd * r * gamma.astype(np.float64)
    m = np.abs(y).max(axis=1, keepdims=True)
    v = y * 127.0 / m
    q_lit = np.clip(np.round(v), -127, 127)
    diff = q.astype(np.float64) - q_lit
    assert np.abs(diff).max() <= 1
    near_tie = np.abs(np.abs(v - np.trunc(v)) - 0.5) < 1e-4
    assert np.all(near_tie[diff != 0])
    assert (diff != 0).mean() < 1e-3
    # dequantization scale: a = max|RMSNorm(x)*gamma| / 127
    assert np.allclose(a, m[:, 0] / 127.0, rtol=1e-6, atol=0)   # max taken over fp32 x*gamma


def pin_ternary_invariants(orc):
    """q in {-1,0,1}; zero fraction of N(0, s^2) latents is erf(sqrt(2/pi)/(2*sqrt(2)))
    = 0.31006 (the mean |w| of a Gaussian is s*sqrt(2/pi)); scaling by 2^k leaves q
    unchanged and scales s by 2^k."""
    rng = np.random.default_rng(13)
    w = rng.standard_normal((2048, 2048)).astype(np.float32) * np.float32(0.02)
    q, s = orc.ternarize(w)
    assert set(np.unique(q).tolist()) <= {-1, 0, 1}
    zf = float((q == 0).mean())
    expect = math.erf(0.5 * math.sqrt(2.0 / math.pi) / math.sqrt(2.0))
    assert abs(zf - expect) < 1e-3, (zf, expect)
    assert abs(s - 0.02 * math.sqrt(2.0 / math.pi)) < 1e-4
    q2, s2 = orc.ternarize(w * np.float32(8.0))
    assert np.array_equal(q, q2) and s2 == s * 8.0
    # absmean is of the whole matrix: a matrix whose rows differ in scale
    w2 = np.array([[4, 4, 4, 4], [0.5, 0.5, -0.5, -0.5]], np.float32)
    q3, s3 = orc.ternarize(w2)
    assert s3 == 2.25 and q3.tolist() == [[1, 1, 1, 1], [0, 0, 0, 0]]


# --------------------------------------------------------------------- BitLinear

def pin_bitlinear_hand(orc):
    """HC7: q_x, q_w, acc and y of a 4-input, 2-output BitLinear worked by hand."""
    g = _golden("bitlinear_hand.json")
    qw, s = orc.ternarize(np.array(g["w_latent"], np.float32))
    assert qw.tolist() == g["q_w"] and s == g["s_w"]
    y, qx, a, acc = orc.bitlinear(np.array([g["x"]], np.float32), qw, s, eps=g["eps"])
    assert qx[0].tolist() == g["q_x"]
    assert acc[0].tolist() == g["acc"]
    assert np.allclose(y[0], g["y"], rtol=1e-13, atol=0), y


def pin_bitlinear_brute(orc):
    """acc equals the fp64 dot of the ternary codes; y stays within the int8 rounding bound
    of the unquantized product RMSNorm(x)*gamma . (q_w*s_w)^T; bias is added."""
    rng = np.random.default_rng(14)
    K, N, M = 512, 96, 40
    x = _bf(rng.standard_normal((M, K)))
    gamma = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    qw, s = orc.ternarize((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    y, qx, a, acc = orc.bitlinear(x, qw, s, gamma=gamma, bias=bias)
    assert np.array_equal(acc, (qx.astype(np.float64) @ qw.astype(np.float64).T).astype(np.int64))
    assert np.all(np.abs(acc) <= 127 * np.count_nonzero(qw, axis=1)[None, :])
    xd = x.astype(np.float64)
    xhat = xd / np.sqrt((xd * xd).mean(axis=1, keepdims=True) + 1e-6) * gamma
    exact = xhat @ (qw.astype(np.float64) * s).T + bias
    bound = s * np.abs(qw).sum(axis=1)[None, :] * np.abs(xhat).max(axis=1, keepdims=True) / 254.0
    assert np.all(np.abs(y - exact) <= bound * (1 + 1e-9) + 1e-12)


# --------------------------------------------------------------------- MLGRU

def pin_recurrence_hand(orc):
    """HC8 (dyadic) and HC9 (closed form h_t = c + f^t (h0 - c)) to T = 32768."""
    g = _golden("recurrence_hand.json")
    f = np.full((1, 3, 1), g["HC8"]["f"])
    c = np.array(g["HC8"]["c"], np.float64).reshape(1, 3, 1)
    h, hl = orc.gated_recurrence(f, c)
    assert h[0, :, 0].tolist() == g["HC8"]["h"] and hl[0, 0] == g["HC8"]["h"][-1]
    T = 32768
    f = np.full((2, T, 3), 0.9)
    c = np.ones((2, T, 3))
    h0 = np.array([[0.0, 2.0, -1.0], [0.5, 0.0, 0.0]])
    h, hl = orc.gated_recurrence(f, c, h0)
    t = np.arange(1, T + 1, dtype=np.float64)[None, :, None]
    closed = 1.0 + 0.9**t * (h0[:, None, :] - 1.0)
    assert np.allclose(h, closed, rtol=1e-12, atol=1e-14)
    for tt, v in g["HC9"]["h"].items():
        assert abs(h[0, int(tt) - 1, 0] - v) < 1e-10


def pin_recurrence_unrolled(orc):
    """Random gates: h_T equals the unrolled sum
    sum_t (prod_{s>t} f_s) (1 - f_t) c_t + (prod_t f_t) h0."""
    rng = np.random.default_rng(15)
    B, T, D = 2, 50, 4
    f = rng.uniform(0.05, 0.99, (B, T, D))
    c = rng.standard_normal((B, T, D))
    h0 = rng.standard_normal((B, D))
    _, hl = orc.gated_recurrence(f, c, h0)
    expect = np.prod(f, axis=1) * h0
    for t in range(T):
        expect = expect + np.prod(f[:, t + 1:, :], axis=1) * (1 - f[:, t, :]) * c[:, t, :]
    assert np.allclose(hl, expect, rtol=1e-12, atol=1e-13)


def pin_mlgru_roles(orc):
    """i_proj feeds the candidate through SiLU and f_proj the forget gate through sigmoid:
    f_pre = 0 (sigmoid 0.5), i_pre = 40 (SiLU = 40 in fp64) gives h = 20, 30, 35."""
    D = 2
    ifg = np.zeros((1, 3, 3 * D))
    ifg[..., :D] = 40.0
    _, hl = orc.mlgru(ifg, gate_mode=1)
    h_seq = []
    for T in (1, 2, 3):
        _, h = orc.mlgru(ifg[:, :T], gate_mode=1)
        h_seq.append(h[0, 0])
    assert h_seq == [20.0, 30.0, 35.0], h_seq
    # forget-gate bias enters the sigmoid: b_f = ln 9 with f_pre = 0 gives f = 0.9
    fb = np.full(D, math.log(9.0), np.float32)
    ifg2 = np.zeros((1, 100, 3 * D))
    ifg2[..., :D] = 40.0
    _, h = orc.mlgru(ifg2, f_bias=fb, gate_mode=1)
    fv = 1.0 / (1.0 + math.exp(-float(np.float32(math.log(9.0)))))
    assert abs(h[0, 0] - 40.0 * (1 - fv**100)) < 1e-9


def pin_mlgru_limits(orc):
    """HC10: f_pre = +40 keeps h = h0 exactly; f_pre = -200 gives h = c = SiLU(i) exactly."""
    D = 3
    h0 = np.array([[1.5, -2.0, 0.25]])
    ifg = np.zeros((1, 7, 3 * D))
    ifg[..., :D] = np.array([0.3, -1.0, 2.0])
    ifg[..., D:2 * D] = 40.0
    _, hl = orc.mlgru(ifg, h0=h0, gate_mode=1)
    assert np.array_equal(hl, h0)
    ifg[..., D:2 * D] = -200.0
    _, hl = orc.mlgru(ifg, h0=h0, gate_mode=1)
    i = np.array([0.3, -1.0, 2.0])
    assert np.allclose(hl[0], i / (1.0 + np.exp(-i)), rtol=4e-16, atol=0)


def pin_output_gate(orc):
    """g_norm: RMSNorm over D of h (a mean, not a sum) times the gain times g*sigmoid(g);
    sigmoid mode: sigmoid(g)*h.  f_pre = -200 makes h = SiLU(i_pre) in one step."""
    D = 4
    ifg = np.zeros((1, 1, 3 * D))
    ifg[0, 0, :D] = [40.0, -40.0, 40.0, -40.0]      # h ~ [40, ~0, 40, ~0]
    ifg[0, 0, D:2 * D] = -200.0
    ifg[0, 0, 2 * D:] = [40.0, 40.0, 0.0, 40.0]
    gw = np.array([2.0, 1.0, 3.0, 0.5], np.float32)
    out, hl = orc.mlgru(ifg, gnorm_w=gw, eps=1e-6, gate_mode=0)
    h = hl[0]
    r = 1.0 / math.sqrt(float(np.mean(h * h)) + 1e-6)
    assert abs(r - 1.0 / math.sqrt(800.0 + 1e-6)) < 1e-15
    expect = h * r * gw * np.array([40.0, 40.0, 0.0, 40.0])
    assert np.allclose(out[0, 0], expect, rtol=1e-14, atol=1e-300)
    out1, _ = orc.mlgru(ifg, gate_mode=1)
    g = ifg[0, 0, 2 * D:]
    assert np.allclose(out1[0, 0], h / (1.0 + np.exp(-g)), rtol=1e-15, atol=0)


def pin_hgrn_lower_bound_gate(orc):
    """Reading R12: f = lb + (1 - lb)*sigmoid(f_pre + b_f).  lb = 0 is the plain MLGRU bit
    for bit; lb = 1 keeps the state exactly (also through a whole block); lb = 0.5 with
    f_pre = 0 gives f = 0.75, so with SiLU(40) = 40 (fp64) and h0 = 0 the state runs
    10, 17.5, 23.125 (dyadic, exact)."""
    D = 2
    rng = np.random.default_rng(19)
    ifg = rng.standard_normal((2, 9, 3 * D))
    fb = np.array([0.3, -0.2], np.float32)
    a, ha = orc.mlgru(ifg, f_bias=fb, gate_mode=0)
    b, hb = orc.mlgru(ifg, f_bias=fb, gate_mode=0, f_lower=np.zeros(D, np.float32))
    assert np.array_equal(a, b) and np.array_equal(ha, hb)
    h0 = rng.standard_normal((2, D))
    _, hl = orc.mlgru(ifg, h0=h0, gate_mode=1, f_lower=np.ones(D, np.float32))
    assert np.array_equal(hl, h0)
    ifg3 = np.zeros((1, 3, 3 * D))
    ifg3[..., :D] = 40.0
    lb = np.full(D, 0.5, np.float32)
    hs = [orc.mlgru(ifg3[:, :T], gate_mode=1, f_lower=lb)[1][0, 0] for T in (1, 2, 3)]
    assert hs == [10.0, 17.5, 23.125], hs
    x = _bf(rng.standard_normal((2, 5, 64)))
    hb0 = rng.standard_normal((2, 64))
    r = orc.block(x, _small_block(orc, 7), h0=hb0, f_lower=np.ones(64, np.float32))
    assert np.array_equal(r["h_last"], hb0)


def pin_hgrn_lower_bounds(orc):
    """Reading R12's bounds: an exclusive cumulative softmax over the layers.  Equal logits
    over 4 layers give 0, 1/4, 1/2, 3/4 exactly; for any logits layer 0 is 0, the bound
    grows with depth and stays below 1, and the last layer's bound is 1 minus the softmax
    weight of the last layer."""
    lb = orc.hgrn_lower_bounds(np.zeros((4, 3), np.float32))
    assert lb.tolist() == [[0.0] * 3, [0.25] * 3, [0.5] * 3, [0.75] * 3], lb.tolist()
    rng = np.random.default_rng(20)
    G = (rng.standard_normal((24, 64)) * 2).astype(np.float32)
    lb = orc.hgrn_lower_bounds(G)
    assert np.all(lb[0] == 0) and np.all(np.diff(lb, axis=0) >= 0) and np.all(lb < 1)
    p = np.exp(G.astype(np.float64))
    p /= p.sum(axis=0)
    assert np.allclose(lb[-1], 1.0 - p[-1], rtol=0, atol=2e-7)
    # a layer whose logit dominates takes nearly all the remaining mass at its successor
    G2 = np.zeros((3, 1), np.float32)
    G2[1, 0] = 30.0
    lb2 = orc.hgrn_lower_bounds(G2)[:, 0]
    assert lb2[0] == 0.0 and float(lb2[1]) < 1e-12 and float(lb2[2]) > 1 - 1e-12


# --------------------------------------------------------------------- GLU / block

def _latent_identity(n, scale):
    return np.eye(n, dtype=np.float32) * np.float32(scale)


def pin_glu_identity(orc):
    """Identity ternary weights reduce the GLU to a closed form.  A latent identity scaled
    by c ternarizes to q = I with s = c/n, so BitLinear(x) = s * a * q_x; the gate branch
    goes through SiLU, the up branch does not."""
    n = 16
    x = np.array([[127, 64, -127, 0, 32, -16, 8, 100, -100, 1, 2, 3, -3, 50, -50, 127]],
                 np.float32) / np.float32(32.0)
    qg, sg = orc.ternarize(_latent_identity(n, 1.0))
    qu, su = orc.ternarize(_latent_identity(n, 2.0))
    qd, sd = orc.ternarize(_latent_identity(n, 4.0))
    assert np.array_equal(qg, np.eye(n)) and sg == 1.0 / n and su == 2.0 / n
    y, m = orc.glu(x, (qg, sg), (qu, su), (qd, sd), eps=1e-6)
    xd = x.astype(np.float64)[0]
    qx = np.clip(np.round(xd * 127.0 / np.abs(xd).max()), -127, 127)   # exact: max is 127/32
    a = (np.abs(xd).max() / 127.0) / math.sqrt(float(np.mean(xd * xd)) + 1e-6)
    vg, vu = qx * a * sg, qx * a * su
    mm = (vg / (1.0 + np.exp(-vg)) * vu).astype(np.float32)
    assert np.allclose(m[0], mm, rtol=1e-6, atol=0)
    md = m[0].astype(np.float64)
    sm = np.float32(127.0) / np.float32(np.abs(m[0]).max())
    qm = np.clip(np.rint(m[0] * sm), -127, 127).astype(np.float64)
    am = (np.abs(md).max() / 127.0) / math.sqrt(float(np.mean(md * md)) + 1e-6)
    assert np.allclose(y[0], qm * am * sd, rtol=1e-6, atol=1e-12)


def _small_block(orc, seed, D=64, F=176, zero=()):
    rng = np.random.default_rng(seed)
    W = {}
    for k, (n, kk) in {"i": (D, D), "f": (D, D), "g": (D, D), "o": (D, D),
                       "gate": (F, D), "up": (F, D), "down": (D, F)}.items():
        lat = (rng.standard_normal((n, kk)) * 0.02).astype(np.float32)
        if k in zero:
            lat[:] = 0.0
        W[k] = orc.ternarize(lat)
    return W


def pin_block_residuals(orc):
    """Zero o_proj weights give y1 = x exactly; zero gate or up weights make the GLU add
    exactly 0; zero i_proj weights give c = SiLU(0) = 0, so h stays 0 and y1 = x."""
    rng = np.random.default_rng(16)
    x = _bf(rng.standard_normal((2, 8, 64)))
    r = orc.block(x, _small_block(orc, 1, zero=("o",)))
    assert np.array_equal(r["y1"], x)
    for z in ("gate", "up"):
        r = orc.block(x, _small_block(orc, 2, zero=(z,)))
        assert np.array_equal(r["y"], r["y1"].astype(np.float64)), z
    r = orc.block(x, _small_block(orc, 3, zero=("i",)))
    assert np.array_equal(r["y1"], x) and not r["h_last"].any()
    r = orc.block(x, _small_block(orc, 4))
    assert not np.array_equal(r["y1"], x) and not np.array_equal(r["y"], r["y1"])


def pin_block_causal_and_carry(orc):
    """Causality: outputs for a prefix do not depend on the suffix.  State carry: running
    T1 + T2 tokens equals running T2 tokens from h0 = h_T1 (bit-exact)."""
    rng = np.random.default_rng(17)
    x = _bf(rng.standard_normal((2, 24, 64)))
    W = _small_block(orc, 5)
    full = orc.block(x, W)
    pre = orc.block(np.ascontiguousarray(x[:, :10]), W)
    assert np.array_equal(full["y"][:, :10], pre["y"])
    post = orc.block(np.ascontiguousarray(x[:, 10:]), W, h0=pre["h_last"])
    assert np.array_equal(full["y"][:, 10:], post["y"])
    assert np.array_equal(full["h_last"], post["h_last"])


def pin_block_stages(orc):
    """Stage records: each BitLinear's recorded q and acc are the quantization and the
    exact integer product of its recorded fp32 input (re-derived here with numpy)."""
    rng = np.random.default_rng(18)
    x = _bf(rng.standard_normal((1, 6, 64)))
    W = _small_block(orc, 6)
    r = orc.block(x, W, record=True)
    cat = {"ifg": np.concatenate([W["i"][0], W["f"][0], W["g"][0]]), "o": W["o"][0],
           "gateup": np.concatenate([W["gate"][0], W["up"][0]]), "down": W["down"][0]}
    for name, st in r["stages"].items():
        xin = st["x_in"].astype(np.float64)
        m = np.abs(xin).max(axis=1, keepdims=True)
        s = (np.float32(127.0) / m.astype(np.float32)).astype(np.float32)
        q = np.clip(np.rint((st["x_in"] * s).astype(np.float32)), -127, 127)
        assert np.array_equal(q, st["q"]), name
        acc = st["q"].astype(np.int64) @ cat[name].astype(np.int64).T
        assert np.array_equal(acc, st["acc"]), name
    assert np.array_equal(r["stages"]["ifg"]["x_in"], x.reshape(6, 64))
    assert np.array_equal(r["stages"]["gateup"]["x_in"], r["y1"].reshape(6, 64))
    # bf16 activations: every tensor one module hands to the next is a bf16 value -- the
    # i/f/g pre-activations, the g_norm output (o_proj's input), y1, the GLU hidden and the
    # block output; with fp32 activations they are fp32 values that are not all bf16
    for v in (r["ifg"].astype(np.float32), r["stages"]["o"]["x_in"], r["y1"],
              r["stages"]["down"]["x_in"], r["y"].astype(np.float32)):
        assert np.array_equal(_bf(v), v)
    assert np.array_equal(r["ifg"], r["ifg"].astype(np.float32).astype(np.float64))
    assert np.array_equal(r["y"], r["y"].astype(np.float32).astype(np.float64))
    r32 = orc.block(x, W, record=True, resid_bf16=False)
    for v in (r32["ifg"].astype(np.float32), r32["stages"]["o"]["x_in"]):
        assert not np.array_equal(_bf(v), v)


def pin_embedding(orc):
    """Ternary embedding: row id of q_E times s_E, rounded to the residual dtype."""
    qe = np.array([[1, 0, -1, 1], [0, 0, 1, -1], [-1, -1, 0, 0]], np.int8)
    s = 0.0123
    x = orc.embedding(qe, s, np.array([2, 0, 2], np.int32), resid_bf16=True)
    sb = float(_bf(np.float32(s)).reshape(-1)[0])
    assert np.array_equal(x, np.array([[-sb, -sb, 0, 0], [sb, 0, -sb, sb], [-sb, -sb, 0, 0]],
                                      np.float32))


def pin_round_bf16(orc):
    """Double -> bf16 rounding is one rounding to nearest-even (checked on values built
    from their bits, including a tie and a value just above a tie)."""
    one = 1.0
    ulp = 2.0**-7
    vals = [one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + 2.0**-40, -(one + ulp / 2),
            3.0e38 * 1.2, 1e-40]
    got = orc.round_bf16(np.array(vals))
    assert got[0] == 1.0 and got[1] == one + 2 * ulp and got[2] == one + ulp
    assert got[3] == -1.0 and math.isinf(got[4])
    assert got[5] == round(1e-40 / 2.0**-133) * 2.0**-133


# ------------------------------------------------------------------- backward
# Reading R14 (straight-through estimator): the gradients are those of a smooth surrogate
# forward in which the quantizers are the identity.  The pins differentiate that surrogate
# numerically (central differences in fp64), so a mistake in the chain rule (a dropped
# term, a wrong sign or index, a transposed operand) shows up against the forward alone.

def _fd(fun, v, idx, h=1e-6):
    """Central difference of scalar fun() with respect to v[idx] (v modified in place)."""
    old = v[idx]
    v[idx] = old + h
    up = fun()
    v[idx] = old - h
    dn = fun()
    v[idx] = old
    return (up - dn) / (2 * h)


def pin_bitlinear_backward_fd(orc):
    """dx, dgamma, db against central differences of the surrogate y = (x*gamma*r) W_hat^T + b,
    r = (mean x^2 + eps)^-1/2, written here in numpy; dw against differences of
    sum dy * (x_hat W^T) in W, x_hat = q_x * a from the (pinned) activation quantizer."""
    rng = np.random.default_rng(7)
    M, K, N, eps = 3, 8, 5, 1e-6
    x = rng.standard_normal((M, K)).astype(np.float32)
    gamma = (1 + 0.3 * rng.standard_normal(K)).astype(np.float32)
    T = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    s = 0.37
    dy = rng.standard_normal((M, N))
    got = orc.bitlinear_backward(x, T, s, dy, gamma=gamma, eps=eps)
    xs, gs, bs = x.astype(np.float64), gamma.astype(np.float64), np.zeros(N)
    What = s * T.astype(np.float64)

    def loss():
        r = 1.0 / np.sqrt((xs**2).mean(axis=1, keepdims=True) + eps)
        return float(np.sum(dy * ((xs * gs * r) @ What.T + bs)))

    for idx in [(0, 0), (1, 3), (2, 7), (0, 5)]:
        fd = _fd(loss, xs, idx)
        assert abs(got["dx"][idx] - fd) <= 1e-6 * (1 + abs(fd)), ("dx", idx, got["dx"][idx], fd)
    for c in [0, 4, 7]:
        fd = _fd(loss, gs, c)
        assert abs(got["dgamma"][c] - fd) <= 1e-6 * (1 + abs(fd)), ("dgamma", c, got["dgamma"][c], fd)
    for j in [0, 4]:
        fd = _fd(loss, bs, j)
        assert abs(got["db"][j] - fd) <= 1e-6 * (1 + abs(fd)), ("db", j)
    q, a, _ = orc.act_quant(x, gamma, eps)
    xh = q.astype(np.float64) * a[:, None]
    Wv = What.copy()
    lw = lambda: float(np.sum(dy * (xh @ Wv.T)))
    for idx in [(0, 0), (4, 7), (2, 3)]:
        fd = _fd(lw, Wv, idx)
        assert abs(got["dw"][idx] - fd) <= 1e-6 * (1 + abs(fd)), ("dw", idx, got["dw"][idx], fd)


def pin_mlgru_backward_fd(orc):
    """d_ifg (i, f, g parts), dh0, dgnorm_w and df_bias against central differences of the
    (pinned) forward: L = sum dout*out + sum dh_last*h_last, both gate modes, with forget
    bias, lower bound, g_norm weight, initial and final state gradients."""
    rng = np.random.default_rng(11)
    B, T, D, eps = 2, 5, 4, 1e-6
    for gate_mode in (0, 1):
        ifg = rng.standard_normal((B, T, 3 * D))
        fb = (0.5 * rng.standard_normal(D)).astype(np.float32)
        lb = (0.3 * rng.random(D)).astype(np.float32)
        gw = (1 + 0.3 * rng.standard_normal(D)).astype(np.float32)
        h0 = rng.standard_normal((B, D))
        dout = rng.standard_normal((B, T, D))
        dl = rng.standard_normal((B, D))
        got = orc.mlgru_backward(ifg, dout, f_bias=fb, h0=h0, gnorm_w=gw, eps=eps,
                                 gate_mode=gate_mode, f_lower=lb, dh_last=dl)

        def loss():
            out, hl = orc.mlgru(ifg, f_bias=fb, h0=h0, gnorm_w=gw, eps=eps,
                                gate_mode=gate_mode, f_lower=lb)
            return float(np.sum(dout * out) + np.sum(dl * hl))

        # f_bias and gnorm_w are fp32 inputs of the oracle, so they are differentiated through
        # exact identities instead (a shift of every f pre-activation of the channel; out is
        # linear in gnorm_w)
        for idx in [(0, 0, 1), (1, 4, 2), (0, 2, D + 1), (1, 0, D + 3), (0, 4, 2 * D), (1, 3, 2 * D + 2),
                    (0, 1, D), (1, 2, 3)]:
            fd = _fd(loss, ifg, idx)
            assert abs(got["d_ifg"][idx] - fd) <= 1e-6 * (1 + abs(fd)), (gate_mode, "d_ifg", idx, got["d_ifg"][idx], fd)
        for idx in [(0, 0), (1, 3)]:
            fd = _fd(loss, h0, idx)
            assert abs(got["dh0"][idx] - fd) <= 1e-6 * (1 + abs(fd)), (gate_mode, "dh0", idx)
        # df_bias: shifting b_f[d] equals shifting every f pre-activation of channel d
        for d in [0, 2]:
            def lb_shift(hh, d=d):
                old = ifg[:, :, D + d].copy()
                ifg[:, :, D + d] += hh
                v = loss()
                ifg[:, :, D + d] = old
                return v
            fd = (lb_shift(1e-6) - lb_shift(-1e-6)) / 2e-6
            assert abs(got["df_bias"][d] - fd) <= 1e-6 * (1 + abs(fd)), (gate_mode, "df_bias", d)
        if gate_mode == 0:
            # dgnorm_w: out is linear in gnorm_w[d], so the derivative is sum dout*out/w
            out, _ = orc.mlgru(ifg, f_bias=fb, h0=h0, gnorm_w=gw, eps=eps, gate_mode=0, f_lower=lb)
            for d in [1, 3]:
                ref = float(np.sum(dout[:, :, d] * out[:, :, d]) / float(gw[d]))
                assert abs(got["dgnorm_w"][d] - ref) <= 1e-9 * (1 + abs(ref)), ("dgnorm_w", d)


def pin_block_backward_ste(orc):
    """Block gradients (R14) against central differences of the block's straight-through
    surrogate at the base point: every BitLinear computes (u(x_in) + delta) W_hat^T + b with
    u = x_in*gamma*r and delta = q*a - u frozen at the base point (the quantizer's error), so
    the surrogate's value there is the quantized forward and its derivatives are the
    straight-through ones, dW included (through q*a); the MLGRU is the pinned fp64 forward;
    residuals and SiLU(gate)*up are written here.  fp32 activations, both gate modes, with
    biases, gains, forget bias and bound, h0 and dh_T."""
    rng = np.random.default_rng(21)
    B, T, D, F, eps = 2, 5, 16, 24, 1e-6
    M = B * T
    shapes = {"i": (D, D), "f": (D, D), "g": (D, D), "o": (D, D), "gate": (F, D), "up": (F, D),
              "down": (D, F)}
    for gm in (0, 1):
        x = rng.standard_normal((B, T, D)).astype(np.float32)
        g_x = (1 + 0.2 * rng.standard_normal(D)).astype(np.float32)
        g_gu = (1 + 0.2 * rng.standard_normal(D)).astype(np.float32)
        W, What, gam, bias = {}, {}, {}, {}
        for k, (n, kk) in shapes.items():
            q, sc = orc.ternarize((0.3 * rng.standard_normal((n, kk))).astype(np.float32))
            gk = g_x if k in ("i", "f", "g") else (g_gu if k in ("gate", "up") else
                                                   (1 + 0.2 * rng.standard_normal(kk)).astype(np.float32))
            bk = (0.1 * rng.standard_normal(n)).astype(np.float32)
            W[k] = (q, sc, gk, bk)
            What[k] = sc * q.astype(np.float64)
            gam[k] = gk.astype(np.float64).copy()
            bias[k] = bk.astype(np.float64).copy()
        fb = (0.3 * rng.standard_normal(D)).astype(np.float32)
        lb = (0.2 * rng.random(D)).astype(np.float32)
        gw = (1 + 0.2 * rng.standard_normal(D)).astype(np.float32)
        h0 = rng.standard_normal((B, D))
        dy = rng.standard_normal((B, T, D))
        dl = rng.standard_normal((B, D))
        kw = dict(f_bias=fb, gnorm_w=gw, eps=eps, gate_mode=gm, f_lower=lb)
        base = orc.block(x, W, resid_bf16=False, h0=h0, record=True, **kw)
        got = orc.block_backward(x, W, dy, resid_bf16=False, h0=h0, dh_last=dl, **kw)

        def delta(st, k):
            xin = st["x_in"].astype(np.float64)
            r = 1.0 / np.sqrt((xin * xin).mean(axis=1, keepdims=True) + eps)
            return st["q"].astype(np.float64) * st["a"][:, None] - xin * gam[k] * r
        st = base["stages"]
        dlt = {"ifg": delta(st["ifg"], "i"), "o": delta(st["o"], "o"), "gu": delta(st["gateup"], "gate"),
               "down": delta(st["down"], "down")}
        xv, h0v = x.astype(np.float64).reshape(M, D).copy(), h0.copy()

        def bl(xin, k, d):
            r = 1.0 / np.sqrt((xin * xin).mean(axis=1, keepdims=True) + eps)
            return (xin * gam[k] * r + d) @ What[k].T + bias[k]

        def forward():
            ifg = np.concatenate([bl(xv, k, dlt["ifg"]) for k in ("i", "f", "g")], axis=1)
            out, hl = orc.mlgru(ifg.reshape(B, T, 3 * D), h0=h0v, **kw)
            y1 = xv + bl(out.reshape(M, D), "o", dlt["o"])
            gg, uu = bl(y1, "gate", dlt["gu"]), bl(y1, "up", dlt["gu"])
            y = y1 + bl(gg / (1.0 + np.exp(-gg)) * uu, "down", dlt["down"])
            return y, hl

        y0, _ = forward()
        assert np.allclose(y0.reshape(B, T, D), base["y"], rtol=1e-5, atol=1e-5), "surrogate != forward"

        def loss():
            y, hl = forward()
            return float(np.sum(dy.reshape(M, D) * y) + np.sum(dl * hl))

        def chk(what, got_v, arr, idx):
            fd = _fd(loss, arr, idx)
            assert abs(got_v - fd) <= 1e-5 * (1 + abs(fd)), (gm, what, idx, got_v, fd)

        for idx in [(0, 0), (3, 7), (9, 15), (5, 2)]:
            chk("dx", got["dx"].reshape(M, D)[idx], xv, idx)
        for idx in [(0, 1), (1, 14)]:
            chk("dh0", got["dh0"][idx], h0v, idx)
        for k in shapes:
            n, kk = shapes[k]
            for idx in [(0, 0), (n - 1, kk - 1), (n // 2, kk // 3)]:
                chk("dw " + k, got["dw"][k][idx], What[k], idx)
            chk("db " + k, got["db"][k][n // 2], bias[k], n // 2)
            chk("dgamma " + k, got["dgamma"][k][kk // 2], gam[k], kk // 2)
        # the forget bias enters as the f projection's bias does
        assert np.allclose(got["df_bias"], got["db"]["f"], rtol=1e-12, atol=1e-12)


PINS = [pin_act_quant_hand, pin_ternarize_hand, pin_pack_format, pin_trit_pack_hand,
        pin_trit_invariants, pin_quant_invariants,
        pin_quant_literal_rmsnorm, pin_ternary_invariants, pin_bitlinear_hand,
        pin_bitlinear_brute, pin_recurrence_hand, pin_recurrence_unrolled, pin_mlgru_roles,
        pin_mlgru_limits, pin_output_gate, pin_hgrn_lower_bound_gate, pin_hgrn_lower_bounds, pin_glu_identity, pin_block_residuals,
        pin_block_causal_and_carry, pin_block_stages, pin_embedding, pin_round_bf16,
        pin_bitlinear_backward_fd, pin_mlgru_backward_fd, pin_block_backward_ste]
