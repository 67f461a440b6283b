"""ctypes binding of the C oracle (mmf_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests, the package smoke check and the benchmark's
CPU-baseline leg; never by the product path.  Arrays are numpy; fp results are fp64.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mmf_oracle.c")
LIB = os.path.join(HERE, "libmmf_oracle.so")

CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11",
          "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (plain C, OpenMP, no FMA contraction, no fast-math)."""
    subprocess.run(["gcc", *CFLAGS, src, "-o", out, "-lm"], check=True)
    return out


class OrcLinear(C.Structure):
    _fields_ = [("q", C.c_void_p), ("scale", C.c_float), ("gamma", C.c_void_p),
                ("bias", C.c_void_p), ("n", C.c_int64), ("k", C.c_int64)]


class OrcStage(C.Structure):
    _fields_ = [("x_in", C.c_void_p), ("q", C.c_void_p), ("a", C.c_void_p),
                ("acc", C.c_void_p)]


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


class Oracle:
    """Numpy-facing wrapper around one loaded copy of the oracle library."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            build(out=path)
        self.lib = C.CDLL(path)
        L = self.lib
        i64, vp, f32, f64, i32 = C.c_int64, C.c_void_p, C.c_float, C.c_double, C.c_int
        L.orc_ternarize.argtypes = [vp, i64, i64, vp, vp]
        L.orc_pack.argtypes = [vp, i64, i64, vp]
        L.orc_unpack.argtypes = [vp, i64, i64, vp]
        L.orc_act_quant.argtypes = [vp, i64, i64, vp, f64, vp, vp, vp]
        L.orc_accumulate.argtypes = [vp, vp, i64, i64, i64, vp]
        L.orc_bitlinear.argtypes = [vp, i64, C.POINTER(OrcLinear), f64, vp, vp, vp, vp]
        L.orc_gated_recurrence.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp]
        L.orc_mlgru.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, f64, i32, vp, vp]
        L.orc_hgrn_lower_bounds.argtypes = [vp, i64, i64, vp]
        L.orc_bitlinear_backward.argtypes = [vp, i64, C.POINTER(OrcLinear), f64, vp, vp, vp, vp, vp]
        L.orc_mlgru_backward.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, f64, i32, vp, vp, vp,
                                         vp, vp, vp]
        L.orc_block_backward.argtypes = [vp, i64, i64, vp, vp, vp, vp, f64, i32, i32, vp, vp, vp,
                                         vp, vp, vp, vp, vp, vp, vp]
        L.orc_trit_row_bytes.argtypes = [i64]
        L.orc_trit_row_bytes.restype = i64
        L.orc_pack_trits.argtypes = [vp, i64, i64, vp]
        L.orc_unpack_trits.argtypes = [vp, i64, i64, vp]
        L.orc_glu.argtypes = [vp, i64, C.POINTER(OrcLinear), C.POINTER(OrcLinear),
                              C.POINTER(OrcLinear), f64, i32, vp, vp]
        L.orc_block.argtypes = ([vp, i64, i64] + [C.POINTER(OrcLinear)] * 7 +
                                [vp, vp, vp, f64, i32, i32, vp, vp, vp, vp, vp] +
                                [C.POINTER(OrcStage)] * 4)
        L.orc_embedding.argtypes = [vp, f32, i64, i64, vp, i64, i32, vp]
        L.orc_round_bf16_array.argtypes = [vp, vp, i64]
        L.orc_round_bf16.argtypes = [f64]
        L.orc_round_bf16.restype = f64
        self._keep = []

    # ------------------------------------------------------------------ threads
    def max_threads(self) -> int:
        return int(self.lib.orc_max_threads())

    def set_threads(self, n: int) -> None:
        self.lib.orc_set_threads(int(n))

    # ------------------------------------------------------------------ weights
    def ternarize(self, w: np.ndarray):
        w = np.ascontiguousarray(w, dtype=np.float32)
        n, k = w.shape
        q = np.empty((n, k), np.int8)
        s = np.zeros(1, np.float32)
        rc = self.lib.orc_ternarize(_p(w), n, k, _p(q), _p(s))
        if rc:
            raise ValueError(f"orc_ternarize failed ({rc})")
        return q, float(s[0])

    def pack(self, q: np.ndarray) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.int8)
        n, k = q.shape
        out = np.empty((n, k // 16), np.uint32)
        rc = self.lib.orc_pack(_p(q), n, k, _p(out))
        if rc:
            raise ValueError(f"orc_pack failed ({rc})")
        return out

    def unpack(self, packed: np.ndarray, k: int) -> np.ndarray:
        packed = np.ascontiguousarray(packed, dtype=np.uint32)
        n = packed.shape[0]
        q = np.empty((n, k), np.int8)
        rc = self.lib.orc_unpack(_p(packed), n, k, _p(q))
        if rc:
            raise ValueError(f"orc_unpack failed ({rc})")
        return q

    def trit_row_bytes(self, k: int) -> int:
        return int(self.lib.orc_trit_row_bytes(k))

    def pack_trits(self, q: np.ndarray) -> np.ndarray:
        """Base-3 packing, 5 trits per byte: [n, k] int8 -> [n, trit_row_bytes(k)] uint8."""
        q = np.ascontiguousarray(q, dtype=np.int8)
        n, k = q.shape
        out = np.empty((n, self.trit_row_bytes(k)), np.uint8)
        rc = self.lib.orc_pack_trits(_p(q), n, k, _p(out))
        if rc:
            raise ValueError(f"orc_pack_trits failed ({rc})")
        return out

    def unpack_trits(self, packed: np.ndarray, k: int) -> np.ndarray:
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        n = packed.shape[0]
        q = np.empty((n, k), np.int8)
        rc = self.lib.orc_unpack_trits(_p(packed), n, k, _p(q))
        if rc:
            raise ValueError(f"orc_unpack_trits failed ({rc})")
        return q

    # -------------------------------------------------------------- activations
    def act_quant(self, x: np.ndarray, gamma=None, eps: float = 1e-6):
        x = np.ascontiguousarray(x, dtype=np.float32)
        k = x.shape[-1]
        m = x.size // k
        q = np.empty(x.shape, np.int8)
        a = np.empty(x.shape[:-1], np.float64)
        rs = np.empty(x.shape[:-1], np.int32)
        g = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.float32)
        self.lib.orc_act_quant(_p(x), m, k, _p(g), eps, _p(q), _p(a), _p(rs))
        return q, a, rs

    def accumulate(self, qx: np.ndarray, qw: np.ndarray) -> np.ndarray:
        qx = np.ascontiguousarray(qx, dtype=np.int8)
        qw = np.ascontiguousarray(qw, dtype=np.int8)
        k = qx.shape[-1]
        m = qx.size // k
        n = qw.shape[0]
        acc = np.empty(qx.shape[:-1] + (n,), np.int32)
        self.lib.orc_accumulate(_p(qx), _p(qw), m, n, k, _p(acc))
        return acc

    def linear(self, q, scale, gamma=None, bias=None) -> OrcLinear:
        q = np.ascontiguousarray(q, dtype=np.int8)
        g = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.float32)
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        self._keep.append((q, g, b))
        return OrcLinear(_p(q), float(scale), _p(g), _p(b), q.shape[0], q.shape[1])

    def bitlinear(self, x, q, scale, gamma=None, bias=None, eps: float = 1e-6):
        """Returns (y fp64 [..., N], q_x int8, a fp64, acc int32)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        lin = self.linear(q, scale, gamma, bias)
        k = x.shape[-1]
        m = x.size // k
        n = lin.n
        y = np.empty(x.shape[:-1] + (n,), np.float64)
        qx = np.empty(x.shape, np.int8)
        a = np.empty(x.shape[:-1], np.float64)
        acc = np.empty(x.shape[:-1] + (n,), np.int32)
        rc = self.lib.orc_bitlinear(_p(x), m, C.byref(lin), eps, _p(y), _p(qx), _p(a), _p(acc))
        if rc:
            raise ValueError(f"orc_bitlinear failed ({rc})")
        return y, qx, a, acc

    # ------------------------------------------------------------------ MLGRU
    def gated_recurrence(self, f, c, h0=None):
        f = np.ascontiguousarray(f, dtype=np.float64)
        c = np.ascontiguousarray(c, dtype=np.float64)
        B, T, D = f.shape
        h = np.empty_like(f)
        hl = np.empty((B, D), np.float64)
        h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
        self.lib.orc_gated_recurrence(_p(f), _p(c), B, T, D, _p(h0), _p(h), _p(hl))
        return h, hl

    def mlgru(self, ifg, f_bias=None, h0=None, gnorm_w=None, eps: float = 1e-6,
              gate_mode: int = 0, f_lower=None):
        ifg = np.ascontiguousarray(ifg, dtype=np.float64)
        B, T, D3 = ifg.shape
        D = D3 // 3
        out = np.empty((B, T, D), np.float64)
        hl = np.empty((B, D), np.float64)
        fb = None if f_bias is None else np.ascontiguousarray(f_bias, dtype=np.float32)
        gw = None if gnorm_w is None else np.ascontiguousarray(gnorm_w, dtype=np.float32)
        h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
        lb = None if f_lower is None else np.ascontiguousarray(f_lower, dtype=np.float32)
        rc = self.lib.orc_mlgru(_p(ifg), B, T, D, _p(fb), _p(lb), _p(h0), _p(gw), eps,
                                gate_mode, _p(out), _p(hl))
        if rc:
            raise ValueError(f"orc_mlgru failed ({rc})")
        return out, hl

    # --------------------------------------------------------------- backward
    def bitlinear_backward(self, x, q, scale, dy, gamma=None, eps: float = 1e-6):
        """Straight-through BitLinear backward (reading R14).  x [M, K] fp32, q [N, K] int8
        ternary, dy [M, N].  Returns dict dx [M, K], dgamma [K], dw [N, K], db [N] (fp64)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        dy = np.ascontiguousarray(dy, dtype=np.float64)
        M, K = x.shape
        lin = self.linear(q, scale, gamma)
        N = lin.n
        out = {"dx": np.empty((M, K)), "dgamma": np.empty(K), "dw": np.empty((N, K)),
               "db": np.empty(N)}
        rc = self.lib.orc_bitlinear_backward(_p(x), M, C.byref(lin), eps, _p(dy), _p(out["dx"]),
                                             _p(out["dgamma"]), _p(out["dw"]), _p(out["db"]))
        if rc:
            raise ValueError(f"orc_bitlinear_backward failed ({rc})")
        return out

    def mlgru_backward(self, ifg, dout, f_bias=None, h0=None, gnorm_w=None, eps: float = 1e-6,
                       gate_mode: int = 0, f_lower=None, dh_last=None):
        """MLGRU + output gate backward (reading R14).  ifg [B, T, 3D], dout [B, T, D].
        Returns dict d_ifg [B, T, 3D], dh0 [B, D], dgnorm_w [D], df_bias [D] (fp64)."""
        ifg = np.ascontiguousarray(ifg, dtype=np.float64)
        dout = np.ascontiguousarray(dout, dtype=np.float64)
        B, T, D3 = ifg.shape
        D = D3 // 3
        fb = None if f_bias is None else np.ascontiguousarray(f_bias, dtype=np.float32)
        gw = None if gnorm_w is None else np.ascontiguousarray(gnorm_w, dtype=np.float32)
        h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
        lb = None if f_lower is None else np.ascontiguousarray(f_lower, dtype=np.float32)
        dl = None if dh_last is None else np.ascontiguousarray(dh_last, dtype=np.float64)
        out = {"d_ifg": np.empty((B, T, 3 * D)), "dh0": np.empty((B, D)),
               "dgnorm_w": np.empty(D), "df_bias": np.empty(D)}
        rc = self.lib.orc_mlgru_backward(_p(ifg), B, T, D, _p(fb), _p(lb), _p(h0), _p(gw), eps,
                                         gate_mode, _p(dout), _p(dl), _p(out["d_ifg"]),
                                         _p(out["dh0"]), _p(out["dgnorm_w"]), _p(out["df_bias"]))
        if rc:
            raise ValueError(f"orc_mlgru_backward failed ({rc})")
        return out

    def block_backward(self, x, W: dict, dy, f_bias=None, gnorm_w=None, eps: float = 1e-6,
                       gate_mode: int = 0, resid_bf16: bool = True, h0=None, f_lower=None,
                       dh_last=None):
        """Block backward (reading R14).  W as for block(); x [B, T, D], dy [B, T, D].
        Returns dict dx, dh0, dgnorm_w, df_bias and per BitLinear name (i, f, g, o, gate, up,
        down) dw[name] [N, K], db[name] [N], dgamma[name] [K] (fp64)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        B, T, D = x.shape
        names = ("i", "f", "g", "o", "gate", "up", "down")
        lins = [self.linear(*W[k]) for k in names]
        arr = (OrcLinear * 7)(*lins)
        ptrs = (C.c_void_p * 7)(*[C.cast(C.byref(arr, i * C.sizeof(OrcLinear)), C.c_void_p) for i in range(7)])
        dyv = np.ascontiguousarray(dy, dtype=np.float64)
        out = {"dx": np.empty((B, T, D)), "dh0": np.empty((B, D)), "dgnorm_w": np.empty(D),
               "df_bias": np.empty(D), "dw": {}, "db": {}, "dgamma": {}}
        for k, ln in zip(names, lins):
            out["dw"][k] = np.empty((ln.n, ln.k))
            out["db"][k] = np.empty(ln.n)
            out["dgamma"][k] = np.empty(ln.k)
        dwp = (C.c_void_p * 7)(*[_p(out["dw"][k]) for k in names])
        dbp = (C.c_void_p * 7)(*[_p(out["db"][k]) for k in names])
        dgp = (C.c_void_p * 7)(*[_p(out["dgamma"][k]) for k in names])
        fb = None if f_bias is None else np.ascontiguousarray(f_bias, dtype=np.float32)
        lb = None if f_lower is None else np.ascontiguousarray(f_lower, dtype=np.float32)
        gw = None if gnorm_w is None else np.ascontiguousarray(gnorm_w, dtype=np.float32)
        h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
        dl = None if dh_last is None else np.ascontiguousarray(dh_last, dtype=np.float64)
        self._keep.append((arr, ptrs, dwp, dbp, dgp))
        rc = self.lib.orc_block_backward(_p(x), B, T, ptrs, _p(fb), _p(lb), _p(gw), eps, gate_mode,
                                         int(resid_bf16), _p(h0), _p(dyv), _p(dl), _p(out["dx"]),
                                         _p(out["dh0"]), dwp, dbp, dgp, _p(out["dgnorm_w"]),
                                         _p(out["df_bias"]))
        if rc:
            raise ValueError(f"orc_block_backward failed ({rc})")
        return out

    # -------------------------------------------------------------------- GLU
    def glu(self, x, gate, up, down, eps: float = 1e-6, act_bf16: bool = False):
        """gate/up/down: (q, scale[, gamma]) tuples.  Returns (y fp64 [M, D], m [M, F]), m
        rounded to the activation dtype (bf16 when act_bf16)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        D = x.shape[-1]
        M = x.size // D
        lg, lu, ld = (self.linear(*gate), self.linear(*up), self.linear(*down))
        y = np.empty(x.shape, np.float64)
        m = np.empty(x.shape[:-1] + (lg.n,), np.float32)
        rc = self.lib.orc_glu(_p(x), M, C.byref(lg), C.byref(lu), C.byref(ld), eps,
                              int(act_bf16), _p(y), _p(m))
        if rc:
            raise ValueError(f"orc_glu failed ({rc})")
        return y, m

    # ------------------------------------------------------------------ block
    def block(self, x, W: dict, f_bias=None, gnorm_w=None, eps: float = 1e-6,
              gate_mode: int = 0, resid_bf16: bool = True, h0=None, record=False,
              f_lower=None):
        """One block forward.  W maps i, f, g, o, gate, up, down -> (q, scale[, gamma]).

        Returns a dict with y (fp64 [B, T, D]), h_last, ifg, y1 and, when record is set,
        per-BitLinear stage records (x_in, q, a, acc) for ifg, o, gateup, down.
        """
        x = np.ascontiguousarray(x, dtype=np.float32)
        B, T, D = x.shape
        M = B * T
        lins = {k: self.linear(*W[k]) for k in ("i", "f", "g", "o", "gate", "up", "down")}
        F = lins["gate"].n
        y = np.empty((B, T, D), np.float64)
        hl = np.empty((B, D), np.float64)
        ifg = np.empty((B, T, 3 * D), np.float64)
        y1 = np.empty((B, T, D), np.float32)
        fb = None if f_bias is None else np.ascontiguousarray(f_bias, dtype=np.float32)
        lb = None if f_lower is None else np.ascontiguousarray(f_lower, dtype=np.float32)
        gw = None if gnorm_w is None else np.ascontiguousarray(gnorm_w, dtype=np.float32)
        h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
        stages = {}
        recs = []
        for name, K, N in (("ifg", D, 3 * D), ("o", D, D), ("gateup", D, 2 * F),
                           ("down", F, D)):
            if record:
                st = dict(x_in=np.empty((M, K), np.float32), q=np.empty((M, K), np.int8),
                          a=np.empty(M, np.float64), acc=np.empty((M, N), np.int32))
                stages[name] = st
                recs.append(OrcStage(_p(st["x_in"]), _p(st["q"]), _p(st["a"]), _p(st["acc"])))
            else:
                recs.append(None)
        rc = self.lib.orc_block(
            _p(x), B, T, *(C.byref(lins[k]) for k in ("i", "f", "g", "o", "gate", "up", "down")),
            _p(fb), _p(lb), _p(gw), eps, gate_mode, int(resid_bf16), _p(h0), _p(hl), _p(y), _p(ifg),
            _p(y1), *(C.byref(r) if r is not None else None for r in recs))
        if rc:
            raise ValueError(f"orc_block failed ({rc})")
        return dict(y=y, h_last=hl, ifg=ifg, y1=y1, stages=stages)

    def hgrn_lower_bounds(self, G):
        """Per-layer forget-gate lower bounds [L, D] from logits G [L, D] (fp32)."""
        G = np.ascontiguousarray(G, dtype=np.float32)
        L, D = G.shape
        lb = np.empty((L, D), np.float32)
        rc = self.lib.orc_hgrn_lower_bounds(_p(G), L, D, _p(lb))
        if rc:
            raise ValueError(f"orc_hgrn_lower_bounds failed ({rc})")
        return lb

    # -------------------------------------------------------------- embedding
    def embedding(self, qe, scale, ids, resid_bf16: bool = True):
        qe = np.ascontiguousarray(qe, dtype=np.int8)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        V, D = qe.shape
        x = np.empty(ids.shape + (D,), np.float32)
        rc = self.lib.orc_embedding(_p(qe), float(scale), V, D, _p(ids), ids.size,
                                    int(resid_bf16), _p(x))
        if rc:
            raise ValueError(f"orc_embedding failed ({rc})")
        return x

    def round_bf16(self, v):
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty_like(v)
        self.lib.orc_round_bf16_array(_p(v), _p(out), v.size)
        return out


_default = None


def get() -> Oracle:
    """Process-wide oracle instance (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
