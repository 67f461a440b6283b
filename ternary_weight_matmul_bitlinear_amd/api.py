"""Python binding of libmmf: argument marshalling around the C ABI of include/mmf.h.

PyTorch provides device memory and the stream; every step of the forward pass runs in
the HIP kernels of libmmf.  Names follow the C entry points.
"""
from __future__ import annotations

import contextlib
import ctypes as C
from dataclasses import dataclass, field

import numpy as np
import torch

from . import _lib as L

_DT = {torch.float32: L.MMF_F32, torch.bfloat16: L.MMF_BF16}


def _dt(t: torch.dtype) -> int:
    if t not in _DT:
        raise TypeError(f"unsupported dtype {t}; use float32 or bfloat16")
    return _DT[t]


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _on(stream):
    """Make `stream` current for the call, so that outputs, workspaces and temporaries come
    from the caching allocator's pool of the stream the kernels run on (a block handed back
    at the end of the call is then reused only by work ordered after these kernels)."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _host(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(C.c_void_p)


# ------------------------------------------------------------------ host weight prep

def quantize_ternary(w: np.ndarray) -> tuple[np.ndarray, float]:
    """Absmean ternarization on the host (mmf_ternary_quantize)."""
    w, wp = _host(w, np.float32)
    n, k = w.shape
    q = np.empty((n, k), np.int8)
    s = np.zeros(1, np.float32)
    L.check("mmf_ternary_quantize",
            L.lib().mmf_ternary_quantize(wp, n, k, q.ctypes.data_as(C.c_void_p),
                                         s.ctypes.data_as(C.c_void_p)))
    return q, float(s[0])


def pack_ternary(q: np.ndarray) -> np.ndarray:
    q, qp = _host(q, np.int8)
    n, k = q.shape
    out = np.empty((n, k // 16), np.uint32)
    L.check("mmf_ternary_pack", L.lib().mmf_ternary_pack(qp, n, k, out.ctypes.data_as(C.c_void_p)))
    return out


def hgrn_lower_bounds(g: np.ndarray) -> np.ndarray:
    """HGRN forget-gate lower bounds [L, D] from per-layer logits [L, D] (mmf_hgrn_lower_bounds)."""
    g, gp = _host(g, np.float32)
    L_, D = g.shape
    lb = np.empty((L_, D), np.float32)
    L.check("mmf_hgrn_lower_bounds",
            L.lib().mmf_hgrn_lower_bounds(gp, L_, D, lb.ctypes.data_as(C.c_void_p)))
    return lb


def unpack_ternary(packed: np.ndarray, k: int) -> np.ndarray:
    packed, pp = _host(packed, np.uint32)
    n = packed.shape[0]
    q = np.empty((n, k), np.int8)
    L.check("mmf_ternary_unpack", L.lib().mmf_ternary_unpack(pp, n, k, q.ctypes.data_as(C.c_void_p)))
    return q


def trit_row_bytes(k: int) -> int:
    return int(L.lib().mmf_trit_row_bytes(k))


def pack_trits(q: np.ndarray) -> np.ndarray:
    """Base-3 packing, five weights per byte (mmf_ternary_pack_trits): [n, k] int8 ->
    [n, trit_row_bytes(k)] uint8."""
    q, qp = _host(q, np.int8)
    n, k = q.shape
    out = np.empty((n, trit_row_bytes(k)), np.uint8)
    L.check("mmf_ternary_pack_trits",
            L.lib().mmf_ternary_pack_trits(qp, n, k, out.ctypes.data_as(C.c_void_p)))
    return out


def unpack_trits(packed: np.ndarray, k: int) -> np.ndarray:
    packed, pp = _host(packed, np.uint8)
    n = packed.shape[0]
    q = np.empty((n, k), np.int8)
    L.check("mmf_ternary_unpack_trits",
            L.lib().mmf_ternary_unpack_trits(pp, n, k, q.ctypes.data_as(C.c_void_p)))
    return q


@dataclass
class TernaryLinear:
    """A BitLinear on the device: packed ternary codes [N][K/16] + absmean scale."""
    packed: torch.Tensor          # int32 view of the uint32 words, [N, K/16]
    scale: float
    K: int
    N: int
    norm_w: torch.Tensor | None = None
    bias: torch.Tensor | None = None
    eps: float = 1e-6

    @classmethod
    def from_latent(cls, w: np.ndarray, device="cuda", norm_w=None, bias=None, eps=1e-6):
        q, s = quantize_ternary(w)
        return cls.from_ternary(q, s, device, norm_w, bias, eps)

    @classmethod
    def from_ternary(cls, q: np.ndarray, scale: float, device="cuda", norm_w=None, bias=None,
                     eps=1e-6):
        packed = pack_ternary(q)
        t = torch.from_numpy(packed.view(np.int32)).to(device)
        nw = None if norm_w is None else torch.as_tensor(norm_w, dtype=torch.float32, device=device)
        b = None if bias is None else torch.as_tensor(bias, dtype=torch.float32, device=device)
        return cls(t, float(scale), q.shape[1], q.shape[0], nw, b, eps)

    def desc(self) -> L.mmf_bitlinear:
        return L.mmf_bitlinear(_ptr(self.packed), self.scale, _ptr(self.norm_w), _ptr(self.bias),
                               self.eps, self.K, self.N)


@dataclass
class TernaryLinearTrits:
    """A BitLinear with base-3 packed weights on the device: [N, trit_row_bytes(K)] uint8."""
    packed: torch.Tensor
    scale: float
    K: int
    N: int
    norm_w: torch.Tensor | None = None
    bias: torch.Tensor | None = None
    eps: float = 1e-6

    @classmethod
    def from_ternary(cls, q: np.ndarray, scale: float, device="cuda", norm_w=None, bias=None,
                     eps=1e-6):
        t = torch.from_numpy(pack_trits(q)).to(device)
        nw = None if norm_w is None else torch.as_tensor(norm_w, dtype=torch.float32, device=device)
        b = None if bias is None else torch.as_tensor(bias, dtype=torch.float32, device=device)
        return cls(t, float(scale), q.shape[1], q.shape[0], nw, b, eps)

    def desc(self) -> L.mmf_bitlinear_trits:
        return L.mmf_bitlinear_trits(_ptr(self.packed), self.scale, _ptr(self.norm_w),
                                     _ptr(self.bias), self.eps, self.K, self.N)


# ------------------------------------------------------------------ captures

@dataclass
class StageCapture:
    """Device buffers recording one BitLinear stage for token rows [row0, row1)."""
    row0: int
    row1: int
    x_in: torch.Tensor
    q: torch.Tensor
    a: torch.Tensor
    acc: torch.Tensor
    y_out: torch.Tensor

    @classmethod
    def alloc(cls, row0, row1, K, N, N_out=None, device="cuda"):
        """Canary-filled buffers (NaN / -128 / INT_MIN) so unwritten entries show."""
        r = row1 - row0
        N_out = N if N_out is None else N_out
        return cls(row0, row1, torch.full((r, K), float("nan"), device=device),
                   torch.full((r, K), -128, dtype=torch.int8, device=device),
                   torch.full((r,), float("nan"), device=device),
                   torch.full((r, N), -2**31, dtype=torch.int32, device=device),
                   torch.full((r, N_out), float("nan"), device=device))

    def desc(self) -> L.mmf_stage_capture:
        return L.mmf_stage_capture(self.row0, self.row1, _ptr(self.x_in), _ptr(self.q),
                                   _ptr(self.a), _ptr(self.acc), _ptr(self.y_out))

    def host(self) -> dict:
        return {k: getattr(self, k).cpu().numpy() for k in ("x_in", "q", "a", "acc", "y_out")}


@dataclass
class BlockCapture:
    ifg: StageCapture
    o: StageCapture
    gateup: StageCapture
    down: StageCapture

    @classmethod
    def alloc(cls, row0, row1, D, F, device="cuda"):
        return cls(StageCapture.alloc(row0, row1, D, 3 * D, 3 * D, device),
                   StageCapture.alloc(row0, row1, D, D, D, device),
                   StageCapture.alloc(row0, row1, D, 2 * F, F, device),
                   StageCapture.alloc(row0, row1, F, D, D, device))

    def desc(self) -> L.mmf_capture:
        return L.mmf_capture(self.ifg.desc(), self.o.desc(), self.gateup.desc(), self.down.desc())


def _empty_stage():
    return L.mmf_stage_capture(0, 0, None, None, None, None, None)


# ------------------------------------------------------------------ forward calls

def set_regime(regime: int) -> int:
    """0 auto, 1 force the weight-streaming kernel, 2 force the MFMA kernels (k-split up to
    64 rows, 128-row tiles above), 3 force the 128-row tiles (test knob)."""
    r = L.lib().mmf_set_regime(int(regime))
    if r < 0:
        L.check("mmf_set_regime", r)
    return r


def _workspace(nbytes: int, device) -> torch.Tensor | None:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def bitlinear_forward(w: TernaryLinear, x: torch.Tensor, out_dtype=None,
                      capture: StageCapture | None = None, stream=None) -> torch.Tensor:
    """y[m, N] = BitLinear(x[m, K]) (bitlinear_forward)."""
    with _on(stream):
        lib = L.lib()
        x = x.contiguous()
        m = x.numel() // w.K
        out_dtype = x.dtype if out_dtype is None else out_dtype
        y = torch.empty(x.shape[:-1] + (w.N,), dtype=out_dtype, device=x.device)
        d = w.desc()
        nb = lib.bitlinear_workspace_bytes(C.byref(d), m)
        ws = _workspace(nb, x.device)
        cap = C.byref(capture.desc()) if capture is not None else None
        L.check("bitlinear_forward",
                lib.bitlinear_forward(C.byref(d), _ptr(x), _dt(x.dtype), m, _ptr(y), _dt(out_dtype),
                                      _ptr(ws), nb, cap, _stream()))
        return y


def bitlinear_forward_trits(w: TernaryLinearTrits, x: torch.Tensor, out_dtype=None,
                            capture: StageCapture | None = None, stream=None) -> torch.Tensor:
    """y[m, N] = BitLinear(x[m, K]) over base-3 packed weights, m <= 16 (bitlinear_forward_trits)."""
    with _on(stream):
        x = x.contiguous()
        m = x.numel() // w.K
        out_dtype = x.dtype if out_dtype is None else out_dtype
        y = torch.empty(x.shape[:-1] + (w.N,), dtype=out_dtype, device=x.device)
        d = w.desc()
        cap = C.byref(capture.desc()) if capture is not None else None
        L.check("bitlinear_forward_trits",
                L.lib().bitlinear_forward_trits(C.byref(d), _ptr(x), _dt(x.dtype), m, _ptr(y),
                                                _dt(out_dtype), cap, _stream()))
        return y


def mlgru_scan(ifg: torch.Tensor, f_bias=None, h0=None, gnorm_w=None, eps: float = 1e-6,
               gate_mode: int = 0, out_dtype=None, h_out: torch.Tensor | None = None,
               stream=None, f_lower=None):
    """MLGRU + output gate over ifg [B, T, 3D] (mlgru_scan).  Returns (out, h_T)."""
    with _on(stream):
        lib = L.lib()
        ifg = ifg.contiguous()
        B, T, D3 = ifg.shape
        D = D3 // 3
        out_dtype = ifg.dtype if out_dtype is None else out_dtype
        out = torch.empty((B, T, D), dtype=out_dtype, device=ifg.device)
        if h_out is None:
            h_out = torch.empty((B, D), dtype=torch.float32, device=ifg.device)
        a = L.mmf_mlgru_args(_ptr(ifg), _dt(ifg.dtype), _ptr(f_bias), _ptr(h0), _ptr(h_out),
                             _ptr(gnorm_w), eps, gate_mode, _ptr(out), _dt(out_dtype), B, T, D,
                             _ptr(f_lower))
        nb = lib.mlgru_workspace_bytes(B, T, D)
        ws = _workspace(nb, ifg.device)
        L.check("mlgru_scan", lib.mlgru_scan(C.byref(a), _ptr(ws), nb, _stream()))
        return out, h_out


def bitlinear_backward(w: TernaryLinear, x: torch.Tensor, dy: torch.Tensor, want_dx: bool = True,
                       want_dgamma: bool = True, want_dw: bool = True, want_db: bool = True,
                       stream=None) -> dict:
    """Straight-through BitLinear backward (bitlinear_backward).  x [m, K] forward input,
    dy [m, N].  Returns dict of fp32 tensors dx [m, K], dgamma [K], dw [N, K], db [N] (the
    ones asked for)."""
    with _on(stream):
        lib = L.lib()
        x = x.contiguous()
        dy = dy.contiguous()
        m = x.numel() // w.K
        dev = x.device
        out = {}
        if want_dx:
            out["dx"] = torch.empty((m, w.K), dtype=torch.float32, device=dev)
        if want_dgamma:
            out["dgamma"] = torch.empty(w.K, dtype=torch.float32, device=dev)
        if want_dw:
            out["dw"] = torch.empty((w.N, w.K), dtype=torch.float32, device=dev)
        if want_db:
            out["db"] = torch.empty(w.N, dtype=torch.float32, device=dev)
        d = w.desc()
        nb = lib.bitlinear_backward_workspace_bytes(C.byref(d), m)
        ws = _workspace(nb, dev)
        L.check("bitlinear_backward",
                lib.bitlinear_backward(C.byref(d), _ptr(x), _dt(x.dtype), m, _ptr(dy), _dt(dy.dtype),
                                       _ptr(out.get("dx")), _ptr(out.get("dgamma")), _ptr(out.get("dw")),
                                       _ptr(out.get("db")), _ptr(ws), nb, _stream()))
        return out


def mlgru_backward(ifg: torch.Tensor, dout: torch.Tensor, f_bias=None, h0=None, gnorm_w=None,
                   eps: float = 1e-6, gate_mode: int = 0, f_lower=None, dh_last=None,
                   stream=None) -> dict:
    """MLGRU + output gate backward (mlgru_backward).  ifg [B, T, 3D], dout [B, T, D].
    Returns dict of fp32 tensors d_ifg [B, T, 3D], dh0 [B, D], dgnorm_w [D], df_bias [D]."""
    with _on(stream):
        lib = L.lib()
        ifg = ifg.contiguous()
        dout = dout.contiguous()
        B, T, D3 = ifg.shape
        D = D3 // 3
        dev = ifg.device
        out = {"d_ifg": torch.empty((B, T, D3), dtype=torch.float32, device=dev),
               "dh0": torch.empty((B, D), dtype=torch.float32, device=dev),
               "dgnorm_w": torch.empty(D, dtype=torch.float32, device=dev),
               "df_bias": torch.empty(D, dtype=torch.float32, device=dev)}
        a = L.mmf_mlgru_args(_ptr(ifg), _dt(ifg.dtype), _ptr(f_bias), _ptr(h0), None,
                             _ptr(gnorm_w), eps, gate_mode, None, _dt(ifg.dtype), B, T, D,
                             _ptr(f_lower))
        nb = lib.mlgru_backward_workspace_bytes(B, T, D)
        ws = _workspace(nb, dev)
        L.check("mlgru_backward",
                lib.mlgru_backward(C.byref(a), _ptr(dout), _dt(dout.dtype), _ptr(dh_last),
                                   _ptr(out["d_ifg"]), _ptr(out["dh0"]), _ptr(out["dgnorm_w"]),
                                   _ptr(out["df_bias"]), _ptr(ws), nb, _stream()))
        return out


BLOCK_LINEARS = ("i", "f", "g", "o", "gate", "up", "down")
BLOCK_GAINS = ("x", "o", "y1", "m")   # inputs of i|f|g, o_proj, gate|up, down


def block_backward(blk: "Block", x: torch.Tensor, dy: torch.Tensor, h0: torch.Tensor | None = None,
                   dh_last: torch.Tensor | None = None, grads=None, stream=None) -> dict:
    """Every gradient of block_forward (block_backward).  x [B, T, D], dy [B, T, D].  Returns
    dict of fp32 tensors: dx [B, T, D], dh0 [B, D], dw[name] [N, K] and db[name] [N] per
    BitLinear, dgamma[input] [K] for the norm gains of x, o, y1 and m, dgnorm_w and df_bias.
    grads: the parameter gradients wanted, as names "dw/<linear>", "db/<linear>",
    "dgamma/<input>", "dgnorm_w", "df_bias" (None: all); the others are not computed and are
    absent from the result."""
    def want(key):
        return grads is None or key in grads

    with _on(stream):
        lib = L.lib()
        x = x.contiguous()
        dy = dy.contiguous()
        B, T, D = x.shape
        dev = x.device
        f32 = dict(dtype=torch.float32, device=dev)
        lins = {k: getattr(blk, k) for k in BLOCK_LINEARS}
        out = {"dx": torch.empty((B, T, D), **f32), "dh0": torch.empty((B, D), **f32),
               "dw": {k: torch.empty((l.N, l.K), **f32) for k, l in lins.items() if want("dw/" + k)},
               "db": {k: torch.empty(l.N, **f32) for k, l in lins.items() if want("db/" + k)},
               "dgamma": {k: torch.empty(n, **f32) for k, n in zip(BLOCK_GAINS, (D, D, D, blk.F))
                          if want("dgamma/" + k)}}
        for k in ("dgnorm_w", "df_bias"):
            if want(k):
                out[k] = torch.empty(D, **f32)
        grads_c = L.mmf_block_grads((C.c_void_p * 7)(*[_ptr(out["dw"].get(k)) for k in BLOCK_LINEARS]),
                                    (C.c_void_p * 7)(*[_ptr(out["db"].get(k)) for k in BLOCK_LINEARS]),
                                    (C.c_void_p * 4)(*[_ptr(out["dgamma"].get(k)) for k in BLOCK_GAINS]),
                                    _ptr(out.get("dgnorm_w")), _ptr(out.get("df_bias")))
        d = blk.desc()
        nb = lib.block_backward_workspace_bytes(C.byref(d), B, T)
        ws = _workspace(nb, dev)
        L.check("block_backward",
                lib.block_backward(C.byref(d), _ptr(x), _dt(x.dtype), B, T, _ptr(h0), _ptr(dy),
                                   _dt(dy.dtype), _ptr(dh_last), _ptr(out["dx"]), _ptr(out["dh0"]),
                                   C.byref(grads_c), _ptr(ws), nb, _stream()))
        return out


def glu_forward(gate: TernaryLinear, up: TernaryLinear, down: TernaryLinear, x: torch.Tensor,
                residual: torch.Tensor | None = None, capture: BlockCapture | None = None,
                stream=None) -> torch.Tensor:
    """y = down(SiLU(gate(x)) * up(x)) (+ residual) (glu_forward)."""
    with _on(stream):
        lib = L.lib()
        x = x.contiguous()
        m = x.numel() // gate.K
        y = torch.empty_like(x)
        dg, du, dd = gate.desc(), up.desc(), down.desc()
        nb = lib.glu_workspace_bytes(C.byref(dg), C.byref(dd), m)
        ws = _workspace(nb, x.device)
        cap = None
        if capture is not None:
            cap = L.mmf_capture(_empty_stage(), _empty_stage(), capture.gateup.desc(), capture.down.desc())
        L.check("glu_forward",
                lib.glu_forward(C.byref(dg), C.byref(du), C.byref(dd), _ptr(x), _dt(x.dtype), m,
                                _ptr(residual.contiguous() if residual is not None else None), _ptr(y),
                                _ptr(ws), nb, C.byref(cap) if cap is not None else None,
                                _stream()))
        return y


@dataclass
class Block:
    """One MatMul-free block: i, f, g, o [D, D]; gate, up [F, D]; down [D, F]."""
    i: TernaryLinear
    f: TernaryLinear
    g: TernaryLinear
    o: TernaryLinear
    gate: TernaryLinear
    up: TernaryLinear
    down: TernaryLinear
    f_bias: torch.Tensor | None = None
    gnorm_w: torch.Tensor | None = None
    eps: float = 1e-6
    gate_mode: int = 0
    f_lower: torch.Tensor | None = None
    _desc: L.mmf_block | None = field(default=None, repr=False)

    @property
    def D(self) -> int:
        return self.i.K

    @property
    def F(self) -> int:
        return self.gate.N

    @classmethod
    def from_latents(cls, lat: dict, device="cuda", f_bias=None, gnorm_w=None, eps=1e-6,
                     gate_mode=0, f_lower=None):
        mats = {k: TernaryLinear.from_latent(lat[k], device, eps=eps)
                for k in ("i", "f", "g", "o", "gate", "up", "down")}
        fb = None if f_bias is None else torch.as_tensor(f_bias, dtype=torch.float32, device=device)
        gw = None if gnorm_w is None else torch.as_tensor(gnorm_w, dtype=torch.float32, device=device)
        lb = None if f_lower is None else torch.as_tensor(f_lower, dtype=torch.float32, device=device)
        return cls(**mats, f_bias=fb, gnorm_w=gw, eps=eps, gate_mode=gate_mode, f_lower=lb)

    def desc(self) -> L.mmf_block:
        if self._desc is None:
            self._desc = L.mmf_block(self.i.desc(), self.f.desc(), self.g.desc(), self.o.desc(),
                                     self.gate.desc(), self.up.desc(), self.down.desc(),
                                     _ptr(self.f_bias), _ptr(self.gnorm_w), self.eps,
                                     self.gate_mode, _ptr(self.f_lower))
        return self._desc


def block_workspace_bytes(block: Block, B: int, T: int) -> int:
    d = block.desc()
    return int(L.lib().block_workspace_bytes(C.byref(d), B, T))


def block_forward(block: Block, x: torch.Tensor, h_state: torch.Tensor | None = None,
                  y: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                  capture: BlockCapture | None = None, stream=None) -> torch.Tensor:
    """One block forward on x [B, T, D] (block_forward); h_state [B, D] fp32 is updated."""
    with _on(stream):
        lib = L.lib()
        B, T, D = x.shape
        if y is None:
            y = torch.empty_like(x)
        d = block.desc()
        nb = lib.block_workspace_bytes(C.byref(d), B, T)
        if ws is None or ws.numel() < nb:
            ws = _workspace(nb, x.device)
        cap = C.byref(capture.desc()) if capture is not None else None
        L.check("block_forward",
                lib.block_forward(C.byref(d), _ptr(x), _dt(x.dtype), B, T, _ptr(h_state), _ptr(y),
                                  _ptr(ws), ws.numel(), cap, _stream()))
        return y


def block_forward_noalloc(block: Block, x: torch.Tensor, h_state: torch.Tensor | None = None,
                          y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """block_forward on the library's static per-GPU scratch (block_forward_noalloc): the
    library allocates nothing; y is allocated here only when the caller passes none."""
    with _on(stream):
        B, T, D = x.shape
        if y is None:
            y = torch.empty_like(x)
        d = block.desc()
        L.check("block_forward_noalloc",
                L.lib().block_forward_noalloc(C.byref(d), _ptr(x), _dt(x.dtype), B, T,
                                              _ptr(h_state), _ptr(y), _stream()))
        return y


def embedding_forward(packed: torch.Tensor, scale: float, vocab: int, D: int,
                      ids: torch.Tensor, dtype=torch.bfloat16, stream=None) -> torch.Tensor:
    with _on(stream):
        x = torch.empty(ids.shape + (D,), dtype=dtype, device=ids.device)
        L.check("embedding_forward",
                L.lib().embedding_forward(_ptr(packed), scale, vocab, D, _ptr(ids), ids.numel(),
                                          _ptr(x), _dt(dtype), _stream()))
        return x


class Stack:
    """L blocks with an optional ternary embedding and head."""

    def __init__(self, blocks: list[Block], embed: TernaryLinear | None = None,
                 head: TernaryLinear | None = None):
        self.blocks = blocks
        self.embed = embed
        self.head = head
        arr = (L.mmf_block * len(blocks))(*[b.desc() for b in blocks])
        self._arr = arr
        self._head = head.desc() if head is not None else None
        self._desc = L.mmf_stack(arr, len(blocks),
                                 _ptr(embed.packed) if embed is not None else None,
                                 embed.scale if embed is not None else 0.0,
                                 embed.N if embed is not None else 0,
                                 C.pointer(self._head) if self._head is not None else None)

    def workspace_bytes(self, B: int, T: int) -> int:
        return int(L.lib().stack_workspace_bytes(C.byref(self._desc), B, T))


def stack_forward(stack: Stack, B: int, T: int, ids: torch.Tensor | None = None,
                  x: torch.Tensor | None = None, h_state: torch.Tensor | None = None,
                  dtype=torch.bfloat16, want_y: bool = True, want_logits: bool = False,
                  ws: torch.Tensor | None = None, y: torch.Tensor | None = None,
                  logits: torch.Tensor | None = None, stream=None):
    """Run the stack (stack_forward).  Returns (y or None, logits or None)."""
    with _on(stream):
        lib = L.lib()
        dev = (ids if ids is not None else x).device
        D = stack.blocks[0].D
        if want_y and y is None:
            y = torch.empty((B, T, D), dtype=dtype, device=dev)
        if want_logits and logits is None:
            logits = torch.empty((B * T, stack.head.N), dtype=torch.float32, device=dev)
        nb = stack.workspace_bytes(B, T)
        if ws is None or ws.numel() < nb:
            ws = _workspace(nb, dev)
        L.check("stack_forward",
                lib.stack_forward(C.byref(stack._desc), _ptr(ids), _ptr(x), _dt(dtype), B, T,
                                  _ptr(h_state), _ptr(y) if want_y else None,
                                  _ptr(logits) if want_logits else None, _ptr(ws), ws.numel(),
                                  _stream()))
        return (y if want_y else None), (logits if want_logits else None)


class DecodeStep:
    """One-launch decode step of a stack for one sequence (stack_decode_*): owns the
    workspace (exchange area and layer table), initialised once for the stack."""

    def __init__(self, stack: Stack, device="cuda", stream=None):
        self.stack = stack
        with _on(stream):
            nb = int(L.lib().stack_decode_workspace_bytes(C.byref(stack._desc)))
            self.ws = torch.empty(nb, dtype=torch.uint8, device=device)
            self.init(stream)

    def init(self, stream=None) -> None:
        with _on(stream):
            L.check("stack_decode_init",
                    L.lib().stack_decode_init(C.byref(self.stack._desc), _ptr(self.ws),
                                              self.ws.numel(), _stream()))

    def step(self, ids: torch.Tensor, h_state: torch.Tensor, logits: torch.Tensor | None = None,
             y: torch.Tensor | None = None, stream=None):
        """ids [1] int32, h_state [L, 1, D] fp32 (updated); returns (logits [1, V] fp32, y)."""
        with _on(stream):
            L.check("stack_decode_step",
                    L.lib().stack_decode_step(C.byref(self.stack._desc), _ptr(ids), _ptr(h_state),
                                              _ptr(logits), _ptr(y), _ptr(self.ws),
                                              self.ws.numel(), _stream()))
            return logits, y

    def status(self, stream=None) -> None:
        with _on(stream):
            L.check("stack_decode_status", L.lib().stack_decode_status(_ptr(self.ws), _stream()))

    def stage_stamps(self) -> torch.Tensor:
        """Workgroup 0's 100 MHz stamps of the last step, [4 * n_layers + 2, 2] int64 (the
        workspace bytes 256 onwards): row 0 the kernel's start, row 4l + k the start and end of
        layer l's wait k (layer input, i|f|g, y1, GLU hidden), row 4 n_layers the head's wait,
        the last row's first entry the end of the work."""
        n = 4 * len(self.stack.blocks) + 2
        return self.ws[256:256 + 16 * n].view(torch.int64).view(n, 2).cpu()


def timing_enable(on: bool = True) -> None:
    L.check("mmf_timing_enable", L.lib().mmf_timing_enable(int(on)))


def timing_families(names=None) -> None:
    """Time only the named kernel families (None: all of them)."""
    if names is None:
        mask = 0xFFFFFFFF
    else:
        lib = L.lib()
        idx = {lib.mmf_timing_name(i).decode(): i for i in range(lib.mmf_timing_count())}
        mask = 0
        for n in names:
            mask |= 1 << idx[n]
    L.check("mmf_timing_families", L.lib().mmf_timing_families(mask))


def timing_reset() -> None:
    L.check("mmf_timing_reset", L.lib().mmf_timing_reset())


def timing_query(family: str) -> tuple[int, float]:
    n = C.c_int64(0)
    ms = C.c_double(0.0)
    L.check("mmf_timing_query",
            L.lib().mmf_timing_query(family.encode(), C.byref(n), C.byref(ms)))
    return int(n.value), float(ms.value)
