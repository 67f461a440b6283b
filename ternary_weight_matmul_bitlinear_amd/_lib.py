"""ctypes declarations of libmmf (include/mmf.h).  Loading fails loudly when the HIP
library has not been built: there is no fallback path."""
from __future__ import annotations

import ctypes as C
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmmf.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "mmf.h")

MMF_F32, MMF_BF16 = 0, 1
GATE_SWISH_RMSNORM, GATE_SIGMOID = 0, 1
STATUS = {0: "MMF_OK", -1: "MMF_EINVAL", -2: "MMF_ESHAPE", -3: "MMF_EALIGN", -4: "MMF_EDTYPE",
          -5: "MMF_EWORKSPACE", -6: "MMF_EHIP", -7: "MMF_EDEVICE"}

vp, i32, i64, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t


class mmf_bitlinear(C.Structure):
    _fields_ = [("packed", vp), ("scale", f32), ("norm_w", vp), ("bias", vp), ("eps", f32),
                ("K", i32), ("N", i32)]


class mmf_block(C.Structure):
    _fields_ = [(n, mmf_bitlinear) for n in ("i", "f", "g", "o", "gate", "up", "down")] + [
        ("f_bias", vp), ("gnorm_w", vp), ("eps", f32), ("gate_mode", i32), ("f_lower", vp)]


class mmf_block_grads(C.Structure):
    _fields_ = [("dw", vp * 7), ("db", vp * 7), ("dgamma", vp * 4), ("dgnorm_w", vp), ("df_bias", vp)]


class mmf_bitlinear_trits(C.Structure):
    _fields_ = [("packed", vp), ("scale", f32), ("norm_w", vp), ("bias", vp), ("eps", f32),
                ("K", i32), ("N", i32)]


class mmf_stage_capture(C.Structure):
    _fields_ = [("row0", i64), ("row1", i64), ("x_in", vp), ("q", vp), ("a", vp), ("acc", vp),
                ("y_out", vp)]


class mmf_capture(C.Structure):
    _fields_ = [(n, mmf_stage_capture) for n in ("ifg", "o", "gateup", "down")]


class mmf_mlgru_args(C.Structure):
    _fields_ = [("ifg", vp), ("ifg_dt", i32), ("f_bias", vp), ("h0", vp), ("h_out", vp),
                ("gnorm_w", vp), ("eps", f32), ("gate_mode", i32), ("out", vp), ("out_dt", i32),
                ("B", i64), ("T", i64), ("D", i64), ("f_lower", vp)]


class mmf_stack(C.Structure):
    _fields_ = [("blocks", C.POINTER(mmf_block)), ("n_layers", i32), ("embed_packed", vp),
                ("embed_scale", f32), ("vocab", i64), ("head", C.POINTER(mmf_bitlinear))]


P = C.POINTER
SIGNATURES = {
    "mmf_abi_version": (C.c_int, []),
    "mmf_last_error": (C.c_char_p, []),
    "mmf_set_regime": (C.c_int, [C.c_int]),
    "mmf_timing_enable": (C.c_int, [C.c_int]),
    "mmf_timing_families": (C.c_int, [C.c_uint32]),
    "mmf_timing_reset": (C.c_int, []),
    "mmf_timing_query": (C.c_int, [C.c_char_p, P(i64), P(C.c_double)]),
    "mmf_timing_name": (C.c_char_p, [C.c_int]),
    "mmf_timing_count": (C.c_int, []),
    "mmf_ternary_quantize": (C.c_int, [vp, i64, i64, vp, vp]),
    "mmf_ternary_pack": (C.c_int, [vp, i64, i64, vp]),
    "mmf_ternary_unpack": (C.c_int, [vp, i64, i64, vp]),
    "mmf_hgrn_lower_bounds": (C.c_int, [vp, i64, i64, vp]),
    "mmf_trit_row_bytes": (i64, [i64]),
    "mmf_ternary_pack_trits": (C.c_int, [vp, i64, i64, vp]),
    "mmf_ternary_unpack_trits": (C.c_int, [vp, i64, i64, vp]),
    "bitlinear_forward_trits": (C.c_int, [P(mmf_bitlinear_trits), vp, C.c_int, i64, vp, C.c_int,
                                          P(mmf_stage_capture), vp]),
    "bitlinear_workspace_bytes": (sz, [P(mmf_bitlinear), i64]),
    "bitlinear_forward": (C.c_int, [P(mmf_bitlinear), vp, C.c_int, i64, vp, C.c_int, vp, sz,
                                    P(mmf_stage_capture), vp]),
    "mlgru_workspace_bytes": (sz, [i64, i64, i64]),
    "mlgru_scan": (C.c_int, [P(mmf_mlgru_args), vp, sz, vp]),
    "glu_workspace_bytes": (sz, [P(mmf_bitlinear), P(mmf_bitlinear), i64]),
    "glu_forward": (C.c_int, [P(mmf_bitlinear), P(mmf_bitlinear), P(mmf_bitlinear), vp, C.c_int,
                              i64, vp, vp, vp, sz, P(mmf_capture), vp]),
    "block_workspace_bytes": (sz, [P(mmf_block), i64, i64]),
    "block_forward": (C.c_int, [P(mmf_block), vp, C.c_int, i64, i64, vp, vp, vp, sz,
                                P(mmf_capture), vp]),
    "block_scratch_bytes": (sz, []),
    "block_forward_noalloc": (C.c_int, [P(mmf_block), vp, C.c_int, i64, i64, vp, vp, vp]),
    "embedding_forward": (C.c_int, [vp, f32, i64, i64, vp, i64, vp, C.c_int, vp]),
    "stack_workspace_bytes": (sz, [P(mmf_stack), i64, i64]),
    "stack_forward": (C.c_int, [P(mmf_stack), vp, vp, C.c_int, i64, i64, vp, vp, vp, vp, sz, vp]),
    "stack_decode_workspace_bytes": (sz, [P(mmf_stack)]),
    "stack_decode_init": (C.c_int, [P(mmf_stack), vp, sz, vp]),
    "stack_decode_step": (C.c_int, [P(mmf_stack), vp, vp, vp, vp, vp, sz, vp]),
    "stack_decode_status": (C.c_int, [vp, vp]),
    "bitlinear_backward_workspace_bytes": (sz, [P(mmf_bitlinear), i64]),
    "bitlinear_backward": (C.c_int, [P(mmf_bitlinear), vp, C.c_int, i64, vp, C.c_int, vp, vp, vp,
                                     vp, vp, sz, vp]),
    "mlgru_backward_workspace_bytes": (sz, [i64, i64, i64]),
    "mlgru_backward": (C.c_int, [P(mmf_mlgru_args), vp, C.c_int, vp, vp, vp, vp, vp, vp, sz, vp]),
    "block_backward_workspace_bytes": (sz, [P(mmf_block), i64, i64]),
    "block_backward": (C.c_int, [P(mmf_block), vp, C.c_int, i64, i64, vp, vp, C.c_int, vp, vp, vp,
                                 P(mmf_block_grads), vp, sz, vp]),
}


def header_functions(path: str = HEADER) -> list[str]:
    """Names of the functions declared in include/mmf.h."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    skip = {"defined", "if", "while", "sizeof"}
    return [n for n in names if n not in skip and not n.isupper()]


_lib = None


class MMFError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} -> {STATUS.get(code, code)}: {msg}")
        self.code = code


def lib(path: str = LIB_PATH) -> C.CDLL:
    """Load libmmf.so once; raise if it is missing (build it with __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"libmmf.so not found at {path}: the HIP library must be built "
                              "first (python -c 'import __graft_entry__ as g; g.build()')")
        L = C.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(fn: str, code: int) -> None:
    if code != 0:
        raise MMFError(fn, code, lib().mmf_last_error().decode())
