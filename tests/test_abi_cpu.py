"""CPU-only checks of the C ABI: the library loads and exports every declared symbol, the
host weight preparation agrees bit for bit with the oracle, and argument validation
returns the documented status before anything is launched."""
import ctypes as C
import subprocess

import numpy as np
import pytest

from ternary_weight_matmul_bitlinear_amd import _lib as L
from ternary_weight_matmul_bitlinear_amd import api


@pytest.fixture(scope="module")
def lib():
    return L.lib()


def test_exports_every_declared_symbol(lib):
    names = L.header_functions()
    assert len(names) >= 20
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(lib, n)
    assert set(L.SIGNATURES) == set(names)


def test_abi_version(lib):
    assert lib.mmf_abi_version() == 2


def test_timing_names(lib):
    names = [lib.mmf_timing_name(i).decode() for i in range(lib.mmf_timing_count())]
    assert "gemm_gateup" in names and "gemv" in names and "scan" in names
    assert lib.mmf_timing_name(99) is None


@pytest.mark.parametrize("seed,shape,std", [(0, (64, 256), 0.02), (1, (300, 512), 1.0),
                                            (2, (7, 16), 0.5), (3, (1024, 2048), 0.02)])
def test_host_ternarize_matches_oracle(orc, seed, shape, std):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(shape) * std).astype(np.float32)
    # plant exact ties at +-0.5 * scale
    q_o, s_o = orc.ternarize(w)
    w.flat[::37] = np.float32(0.5) * np.float32(s_o)
    q_o, s_o = orc.ternarize(w)
    q_l, s_l = api.quantize_ternary(w)
    assert s_l == s_o
    assert np.array_equal(q_l, q_o)


def test_host_ternarize_hand_cases():
    q, s = api.quantize_ternary(np.array([[0.5, -0.25, 0, 1.5], [-1, 0.125, 0.375, -0.25]],
                                         np.float32))
    assert s == 0.5 and q.tolist() == [[1, 0, 0, 1], [-1, 0, 1, 0]]
    q, s = api.quantize_ternary(np.zeros((2, 16), np.float32))
    assert s == np.float32(1e-5) and not q.any()


def test_pack_matches_oracle_and_roundtrips(orc):
    rng = np.random.default_rng(5)
    q = rng.integers(-1, 2, size=(33, 256)).astype(np.int8)
    p_l = api.pack_ternary(q)
    p_o = orc.pack(q)
    assert np.array_equal(p_l, p_o)
    assert np.array_equal(api.unpack_ternary(p_l, 256), q)
    # the documented example word
    row = np.array([[1, 0, -1, 1, 0, 0, 0, 0, -1, -1, -1, -1, 1, 1, 1, 1]], np.int8)
    assert int(api.pack_ternary(row)[0, 0]) == 0x86848586


def test_pack_unpack_errors(lib):
    with pytest.raises(L.MMFError) as e:
        api.unpack_ternary(np.array([[0x55555557]], np.uint32), 16)
    assert e.value.code == -1
    with pytest.raises(L.MMFError) as e:
        api.pack_ternary(np.array([[2] + [0] * 15], np.int8))
    assert e.value.code == -1
    with pytest.raises(L.MMFError) as e:
        api.pack_ternary(np.zeros((1, 10), np.int8))
    assert e.value.code == -2


FAKE = 0x10000  # an aligned address that is never dereferenced: validation fails first


def _bl(K=256, N=128, packed=FAKE, eps=1e-6):
    return L.mmf_bitlinear(packed, 0.02, None, None, eps, K, N)


def test_bitlinear_validation_codes(lib):
    f = lib.bitlinear_forward
    st = None
    assert f(None, FAKE, 0, 4, FAKE, 0, FAKE, 1 << 20, None, st) == -1
    assert f(C.byref(_bl(packed=0)), FAKE, 0, 4, FAKE, 0, FAKE, 1 << 20, None, st) == -1
    assert f(C.byref(_bl(K=100)), FAKE, 0, 4, FAKE, 0, FAKE, 1 << 20, None, st) == -2
    assert f(C.byref(_bl(packed=FAKE + 4)), FAKE, 0, 4, FAKE, 0, FAKE, 1 << 20, None, st) == -3
    assert f(C.byref(_bl()), FAKE, 7, 4, FAKE, 0, FAKE, 1 << 20, None, st) == -4
    assert f(C.byref(_bl()), FAKE + 8, 0, 4, FAKE, 0, FAKE, 1 << 20, None, st) == -3
    assert f(C.byref(_bl()), None, 0, 4, FAKE, 0, FAKE, 1 << 20, None, st) == -1
    assert f(C.byref(_bl()), FAKE, 0, -1, FAKE, 0, FAKE, 1 << 20, None, st) == -2
    # m == 0 is a no-op that needs no device
    assert f(C.byref(_bl()), None, 0, 0, None, 0, None, 0, None, st) == 0
    assert lib.mmf_last_error() == b"bitlinear_forward: m=-1"  # last non-zero status


def test_workspace_too_small_is_reported(lib):
    prev = lib.mmf_set_regime(2)  # prefill needs the workspace
    try:
        need = lib.bitlinear_workspace_bytes(C.byref(_bl()), 512)
        assert need >= 512 * 256
        rc = lib.bitlinear_forward(C.byref(_bl()), FAKE, 0, 512, FAKE, 0, FAKE, need - 1, None, None)
        assert rc == -5
        assert b"workspace" in lib.mmf_last_error()
    finally:
        lib.mmf_set_regime(prev)


def test_regime_knob(lib):
    assert lib.mmf_set_regime(4) == -1
    prev = lib.mmf_set_regime(1)
    assert lib.mmf_set_regime(prev) == 1


def _block(D=256, F=704, **kw):
    mk = lambda K, N: _bl(K=K, N=N)
    b = L.mmf_block(mk(D, D), mk(D, D), mk(D, D), mk(D, D), mk(D, F), mk(D, F), mk(F, D),
                    None, None, 1e-6, 0)
    for k, v in kw.items():
        setattr(b, k, v)
    return b


def test_block_validation_codes(lib):
    f = lib.block_forward
    ws = 1 << 30
    assert f(None, FAKE, 1, 1, 64, None, FAKE, FAKE, ws, None, None) == -1
    assert f(C.byref(_block(gate_mode=5)), FAKE, 1, 1, 64, None, FAKE, FAKE, ws, None, None) == -1
    b = _block()
    b.o = _bl(K=256, N=128)
    assert f(C.byref(b), FAKE, 1, 1, 64, None, FAKE, FAKE, ws, None, None) == -2
    b = _block()
    b.down = _bl(K=512, N=256)
    assert f(C.byref(b), FAKE, 1, 1, 64, None, FAKE, FAKE, ws, None, None) == -2
    b = _block()
    b.f.norm_w = FAKE
    assert f(C.byref(b), FAKE, 1, 1, 64, None, FAKE, FAKE, ws, None, None) == -1
    assert f(C.byref(_block(D=8192, F=704)), FAKE, 1, 1, 64, None, FAKE, FAKE, ws, None, None) == -2
    assert f(C.byref(_block()), FAKE, 3, 1, 64, None, FAKE, FAKE, ws, None, None) == -4
    need = lib.block_workspace_bytes(C.byref(_block()), 1, 64)
    assert f(C.byref(_block()), FAKE, 1, 1, 64, None, FAKE, FAKE, need - 1, None, None) == -5
    assert f(C.byref(_block()), FAKE, 1, 1, 64, None, FAKE, FAKE + 8, need, None, None) == -3
    assert f(C.byref(_block()), None, 1, 0, 64, None, None, None, 0, None, None) == 0
    # state and per-channel vectors are read 16 bytes at a time
    h_bad = FAKE + 4
    assert f(C.byref(_block()), FAKE, 1, 1, 64, h_bad, FAKE, FAKE, ws, None, None) == -3
    b = _block()
    b.f_bias = h_bad
    assert f(C.byref(b), FAKE, 1, 1, 64, None, FAKE, FAKE, ws, None, None) == -3
    b = _block()
    b.gnorm_w = h_bad
    assert f(C.byref(b), FAKE, 1, 1, 64, None, FAKE, FAKE, ws, None, None) == -3
    cap = L.mmf_capture(L.mmf_stage_capture(5, 2, None, None, None, None, None),
                        *[L.mmf_stage_capture(0, 0, None, None, None, None, None)] * 3)
    assert f(C.byref(_block()), FAKE, 1, 1, 64, None, FAKE, FAKE, ws, C.byref(cap), None) == -1


def test_mlgru_and_glu_validation_codes(lib):
    a = L.mmf_mlgru_args(FAKE, 0, None, None, None, None, 1e-6, 0, FAKE, 0, 2, 64, 100)
    assert lib.mlgru_scan(C.byref(a), FAKE, 1 << 20, None) == -2
    a.D = 256
    a.gate_mode = 4
    assert lib.mlgru_scan(C.byref(a), FAKE, 1 << 20, None) == -1
    a.gate_mode = 0
    a.out_dt = 9
    assert lib.mlgru_scan(C.byref(a), FAKE, 1 << 20, None) == -4
    a.out_dt = 0
    need = lib.mlgru_workspace_bytes(2, 64, 256)
    assert need > 0
    assert lib.mlgru_scan(C.byref(a), FAKE, need - 1, None) == -5
    a.h0 = FAKE + 4
    assert lib.mlgru_scan(C.byref(a), FAKE, need, None) == -3
    a.h0 = None
    g, u, d = _bl(256, 704), _bl(256, 704), _bl(704, 256)
    assert lib.glu_forward(C.byref(g), C.byref(u), C.byref(_bl(512, 256)), FAKE, 0, 4, None, FAKE,
                           FAKE, 1 << 20, None, None) == -2
    u2 = _bl(256, 704)
    u2.eps = 1e-5
    assert lib.glu_forward(C.byref(g), C.byref(u2), C.byref(d), FAKE, 0, 4, None, FAKE,
                           FAKE, 1 << 20, None, None) == -1


def test_no_device_is_an_error_not_a_crash(lib):
    """On a host without a GPU a valid call reports MMF_EHIP/MMF_EDEVICE."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    rc = lib.bitlinear_forward(C.byref(_bl()), FAKE, 0, 4, FAKE, 0, FAKE, 1 << 20, None, None)
    assert rc in (-6, -7)


@pytest.mark.parametrize("L_,D,scale", [(4, 3, 0.0), (24, 64, 2.0), (32, 2560, 1.0)])
def test_host_hgrn_lower_bounds_match_oracle(orc, L_, D, scale):
    """The library's host bound builder and the oracle's agree bit for bit (both sum in
    double in the same order); equal logits give l / L."""
    g = (np.random.default_rng(L_ + D).standard_normal((L_, D)) * scale).astype(np.float32)
    lb = api.hgrn_lower_bounds(g)
    assert np.array_equal(lb, orc.hgrn_lower_bounds(g))
    if scale == 0.0:
        assert np.array_equal(lb, np.repeat((np.arange(L_) / L_)[:, None], D, 1).astype(np.float32))


def test_hgrn_lower_bounds_validation(lib):
    g = np.zeros((2, 4), np.float32)
    out = np.zeros((2, 4), np.float32)
    vp = C.c_void_p
    assert lib.mmf_hgrn_lower_bounds(None, 2, 4, out.ctypes.data_as(vp)) == -1
    assert lib.mmf_hgrn_lower_bounds(g.ctypes.data_as(vp), 0, 4, out.ctypes.data_as(vp)) == -2


@pytest.mark.parametrize("k", [16, 64, 80, 2048, 5632])
def test_host_trit_pack_matches_oracle(orc, k):
    """The library's base-3 packing equals the oracle's byte for byte; the library's unpack
    (fixed-point digit extraction) inverts it; invalid bytes and padding are rejected."""
    q = np.random.default_rng(k).integers(-1, 2, (19, k)).astype(np.int8)
    p = api.pack_trits(q)
    assert api.trit_row_bytes(k) == orc.trit_row_bytes(k)
    assert np.array_equal(p, orc.pack_trits(q))
    assert np.array_equal(api.unpack_trits(p, k), q)
    bad = p.copy()
    bad[3, 0] = 1                     # no group of five trits packs to 1
    with pytest.raises(L.MMFError):
        api.unpack_trits(bad, k)
    with pytest.raises(L.MMFError):
        api.pack_trits(np.full((1, k), 2, np.int8))


def test_lower_bound_trit_and_noalloc_validation_codes(lib):
    """f_lower is read 16 bytes at a time; the trit BitLinear takes 0..16 rows and K a
    multiple of 64 up to 10240; block_forward_noalloc rejects work beyond its static scratch
    before touching the device."""
    b = _block()
    b.f_lower = FAKE + 4
    assert lib.block_forward(C.byref(b), FAKE, 1, 1, 64, None, FAKE, FAKE, 1 << 30, None, None) == -3
    a = L.mmf_mlgru_args(FAKE, 0, None, None, None, None, 1e-6, 0, FAKE, 0, 2, 64, 256, FAKE + 4)
    assert lib.mlgru_scan(C.byref(a), FAKE, 1 << 30, None) == -3
    t = L.mmf_bitlinear_trits(FAKE, 0.5, None, None, 1e-6, 256, 64)
    f = lib.bitlinear_forward_trits
    assert f(C.byref(t), FAKE, 0, 17, FAKE, 0, None, None) == -2
    assert f(C.byref(t), FAKE, 0, 0, FAKE, 0, None, None) == 0
    assert f(C.byref(t), FAKE + 8, 0, 2, FAKE, 0, None, None) == -3
    assert f(C.byref(t), FAKE, 7, 2, FAKE, 0, None, None) == -4
    for K in (100, 10304):
        t.K = K
        assert f(C.byref(t), FAKE, 0, 2, FAKE, 0, None, None) == -2
    big = _block(D=2048, F=5632)
    assert lib.block_workspace_bytes(C.byref(big), 1, 4096) > lib.block_scratch_bytes()
    assert lib.block_forward_noalloc(C.byref(big), FAKE, 1, 1, 4096, None, FAKE, None) == -5
    assert lib.block_forward_noalloc(C.byref(big), FAKE, 1, 0, 4096, None, FAKE, None) == 0


def test_backward_validation_codes(lib):
    f = lib.bitlinear_backward
    args = lambda w, x=FAKE, xdt=0, m=4, dy=FAKE, dydt=0, ws=FAKE, nb=1 << 24: (
        C.byref(w) if w is not None else None, x, xdt, m, dy, dydt, FAKE, FAKE, FAKE, FAKE, ws, nb, None)
    assert f(*args(None)) == -1
    assert f(*args(_bl(K=100))) == -2
    assert f(*args(_bl(256, 100))) == -2                 # N % 8
    assert f(*args(_bl(8256, 64))) == -2                 # K > 8192
    assert f(*args(_bl(), xdt=7)) == -4
    assert f(*args(_bl(), x=FAKE + 8)) == -3
    assert f(*args(_bl(), dy=None)) == -1
    assert f(*args(_bl(), m=-1)) == -2
    need = lib.bitlinear_backward_workspace_bytes(C.byref(_bl()), 4)
    assert need >= 4 * 256 * 5
    assert f(*args(_bl(), nb=need - 1)) == -5
    # m == 0 with no outputs asked for needs no device
    assert f(C.byref(_bl()), None, 0, 0, None, 0, None, None, None, None, None, 0, None) == 0
    g = lib.mlgru_backward
    a = L.mmf_mlgru_args(FAKE, 0, None, None, None, None, 1e-6, 0, None, 0, 2, 64, 100)
    assert g(C.byref(a), FAKE, 0, None, FAKE, None, None, None, FAKE, 1 << 24, None) == -2
    a.D = 256
    a.gate_mode = 4
    assert g(C.byref(a), FAKE, 0, None, FAKE, None, None, None, FAKE, 1 << 24, None) == -1
    a.gate_mode = 0
    assert g(C.byref(a), FAKE, 9, None, FAKE, None, None, None, FAKE, 1 << 24, None) == -4
    assert g(C.byref(a), None, 0, None, FAKE, None, None, None, FAKE, 1 << 24, None) == -1
    a.h0 = FAKE + 4
    assert g(C.byref(a), FAKE, 0, None, FAKE, None, None, None, FAKE, 1 << 24, None) == -3
    a.h0 = None
    assert lib.mlgru_backward_workspace_bytes(2, 64, 256) > lib.mlgru_workspace_bytes(2, 64, 256)
