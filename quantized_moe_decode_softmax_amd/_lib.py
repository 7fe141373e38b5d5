"""ctypes binding of libmoe.so (include/moe_decode.h). Argument marshalling only.

Every function here has the name of the C entry point it calls. Device
buffers are passed as integer addresses (for a torch tensor:
``t.data_ptr()``), streams as integer hipStream_t handles (for torch:
``torch.cuda.current_stream().cuda_stream``). Errors raise ``MoeError`` with
the library's message. There is no fallback: if libmoe.so is missing the
import of this module's functions fails with an explanation.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "moe_decode.h")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_ALIGNMENT = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5
MOE_ERR_TIMEOUT = -6

MOE_PATH_DEFAULT = 0
MOE_PATH_PER_LAYER = 1
MOE_PATH_NO_MFMA = 2

c_i32, c_i64, c_u64, c_f32, c_vp, c_sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float,
                                         ctypes.c_void_p, ctypes.c_size_t)


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (code {code})")
        self.code = code


class moe_shape_t(ctypes.Structure):
    _fields_ = [
        ("hidden", c_i32),
        ("n_experts", c_i32),
        ("inter", c_i32),
        ("top_k", c_i32),
        ("shared_inter", c_i32),
        ("router_bits", c_i32),
        ("expert_bits", c_i32),
        ("shared_bits", c_i32),
        ("group", c_i32),
        ("rms_eps", c_f32),
    ]


class moe_layer_layout_t(ctypes.Structure):
    _fields_ = [(n, c_i64) for n in ("router", "gatevec", "shared", "shared_up", "shared_down", "expert0",
                                      "expert_stride", "expert_up", "expert_down", "total_bytes")]


class moe_stack_t(ctypes.Structure):
    _fields_ = [
        ("shape", moe_shape_t),
        ("n_layers", c_i32),
        ("t_max", c_i32),
        ("flags", c_i32),
        ("magic", ctypes.c_uint32),
        ("ws_dev", c_vp),
        ("ws_bytes", c_sz),
        ("table_offset", c_i64),
        ("reserved", c_i64 * 4),
    ]


class moe_gemv_mat_t(ctypes.Structure):
    _fields_ = [("w_dev", c_vp), ("rows", c_i32), ("reserved", c_i32), ("y_dev", c_vp)]


class moe_attn_shape_t(ctypes.Structure):
    _fields_ = [("n_q", c_i32), ("n_kv", c_i32), ("head_dim", c_i32), ("max_seq", c_i32)]


class moe_gdn_shape_t(ctypes.Structure):
    _fields_ = [("n_k", c_i32), ("n_v", c_i32), ("d_k", c_i32), ("d_v", c_i32)]


_lib: Optional[ctypes.CDLL] = None


def use_library(path: str) -> None:
    """Selects another build of the library (e.g. the phase-trace build
    libmoe_trace.so) before its first use in this process."""
    global LIB_PATH
    if _lib is not None and os.path.abspath(path) != os.path.abspath(LIB_PATH):
        raise RuntimeError("the library is already loaded")
    LIB_PATH = path


def lib() -> ctypes.CDLL:
    """Loads libmoe.so (built by ``python -m quantized_moe_decode_softmax_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m quantized_moe_decode_softmax_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        sp = ctypes.POINTER(moe_shape_t)
        L.moe_matrix_bytes.argtypes = [c_i32, c_i32, c_i32]
        L.moe_matrix_bytes.restype = c_i64
        L.moe_validate_shape.argtypes = [sp]
        L.moe_validate_shape.restype = c_i32
        L.moe_layer_layout.argtypes = [sp, ctypes.POINTER(moe_layer_layout_t)]
        L.moe_layer_layout.restype = c_i32
        L.moe_validate.argtypes = [sp, c_i32]
        L.moe_validate.restype = c_i32
        L.moe_expert_bytes.argtypes = [sp]
        L.moe_expert_bytes.restype = c_i64
        L.moe_layer_bytes.argtypes = [sp]
        L.moe_layer_bytes.restype = c_i64
        L.moe_workspace_bytes.argtypes = [sp, c_i32, c_i32]
        L.moe_workspace_bytes.restype = c_i64
        L.moe_pack_matrix.argtypes = [c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]
        L.moe_pack_matrix.restype = c_i32
        L.moe_unpack_matrix.argtypes = [c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]
        L.moe_unpack_matrix.restype = c_i32
        L.moe_generate_layer.argtypes = [sp, c_u64, c_i32, c_vp, c_vp]
        L.moe_generate_layer.restype = c_i32
        L.moe_generate_rows.argtypes = [c_u64, c_i32, c_i32, c_vp, c_vp]
        L.moe_generate_rows.restype = c_i32
        L.moe_decode_layer.argtypes = [sp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]
        L.moe_decode_layer.restype = c_i32
        L.moe_decode_stack.argtypes = [sp, ctypes.POINTER(c_vp), c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                       c_sz, c_vp]
        L.moe_decode_stack.restype = c_i32
        stp = ctypes.POINTER(moe_stack_t)
        L.moe_stack_init.argtypes = [stp, sp, ctypes.POINTER(c_vp), c_i32, c_i32, c_i32, c_vp, c_sz, c_vp]
        L.moe_stack_init.restype = c_i32
        L.moe_stack_decode.argtypes = [stp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]
        L.moe_stack_decode.restype = c_i32
        L.moe_decode_stack_static.argtypes = [sp, ctypes.POINTER(c_vp), c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp,
                                              c_vp]
        L.moe_decode_stack_static.restype = c_i32
        L.moe_gemv.argtypes = [c_i32, c_i32, c_i32, c_vp, ctypes.POINTER(moe_gemv_mat_t), c_i32, c_vp]
        L.moe_gemv.restype = c_i32
        L.moe_generate_matrix.argtypes = [c_i32, c_i32, c_i32, c_u64, c_i32, c_i32, c_vp, c_vp]
        L.moe_generate_matrix.restype = c_i32
        ap = ctypes.POINTER(moe_attn_shape_t)
        L.moe_gqa_workspace_bytes.argtypes = [ap, c_i32]
        L.moe_gqa_workspace_bytes.restype = c_i64
        L.moe_gqa_decode.argtypes = [ap, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]
        L.moe_gqa_decode.restype = c_i32
        L.moe_gdn_step.argtypes = [ctypes.POINTER(moe_gdn_shape_t), c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                   c_vp]
        L.moe_gdn_step.restype = c_i32
        L.moe_stack_status.argtypes = [sp, c_i32, c_vp, ctypes.POINTER(ctypes.c_uint32), c_vp]
        L.moe_stack_status.restype = c_i32
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_version.argtypes = []
        L.moe_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def header_functions() -> Sequence[str]:
    """Names of the functions include/moe_decode.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def _check(rc: int) -> int:
    if rc < 0:
        raise MoeError(rc, lib().moe_last_error().decode())
    return rc


def make_shape(hidden: int, n_experts: int, inter: int, top_k: int, shared_inter: int, router_bits: int,
               expert_bits: int, shared_bits: int, group: int = 64, rms_eps: float = 1e-6) -> moe_shape_t:
    return moe_shape_t(hidden, n_experts, inter, top_k, shared_inter, router_bits, expert_bits, shared_bits, group,
                       rms_eps)


def _p(x) -> Optional[int]:
    return None if x is None or x == 0 else int(x)


# ------------------------------------------------------------------ entry points
def moe_matrix_bytes(bits: int, rows: int, cols: int) -> int:
    return _check(lib().moe_matrix_bytes(bits, rows, cols))


def moe_validate_shape(shape: moe_shape_t) -> int:
    return _check(lib().moe_validate_shape(ctypes.byref(shape)))


def moe_layer_layout(shape: moe_shape_t) -> Dict[str, int]:
    out = moe_layer_layout_t()
    _check(lib().moe_layer_layout(ctypes.byref(shape), ctypes.byref(out)))
    return {n: getattr(out, n) for n, _ in moe_layer_layout_t._fields_}


def moe_validate(shape: moe_shape_t, T: int) -> int:
    return _check(lib().moe_validate(ctypes.byref(shape), T))


def moe_expert_bytes(shape: moe_shape_t) -> int:
    return _check(lib().moe_expert_bytes(ctypes.byref(shape)))


def moe_layer_bytes(shape: moe_shape_t) -> int:
    return _check(lib().moe_layer_bytes(ctypes.byref(shape)))


def moe_workspace_bytes(shape: moe_shape_t, n_layers: int, T: int) -> int:
    return _check(lib().moe_workspace_bytes(ctypes.byref(shape), n_layers, T))


def moe_pack_matrix(bits: int, codes: np.ndarray, scale_bits: np.ndarray, bias_bits: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    rows, cols = codes.shape
    scale_bits = np.ascontiguousarray(scale_bits, dtype=np.uint16)
    bias_bits = np.ascontiguousarray(bias_bits, dtype=np.uint16)
    if scale_bits.shape != (rows, cols // 64) or bias_bits.shape != (rows, cols // 64):
        raise ValueError("scale/bias must be [rows, cols/64]")
    out = np.empty(moe_matrix_bytes(bits, rows, cols), dtype=np.uint8)
    _check(lib().moe_pack_matrix(bits, rows, cols, codes.ctypes.data, scale_bits.ctypes.data, bias_bits.ctypes.data,
                                 out.ctypes.data))
    return out


def moe_unpack_matrix(bits: int, rows: int, cols: int, packed: np.ndarray):
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    if packed.size < moe_matrix_bytes(bits, rows, cols):
        raise ValueError("packed buffer too small")
    codes = np.empty((rows, cols), dtype=np.uint8)
    sc = np.empty((rows, cols // 64), dtype=np.uint16)
    bi = np.empty((rows, cols // 64), dtype=np.uint16)
    _check(lib().moe_unpack_matrix(bits, rows, cols, packed.ctypes.data, codes.ctypes.data, sc.ctypes.data,
                                   bi.ctypes.data))
    return codes, sc, bi


def moe_generate_layer(shape: moe_shape_t, seed: int, layer: int, layer_dev: int, stream: int = 0) -> None:
    _check(lib().moe_generate_layer(ctypes.byref(shape), seed, layer, _p(layer_dev), _p(stream)))


def moe_generate_rows(seed_x: int, T: int, H: int, out_dev: int, stream: int = 0) -> None:
    _check(lib().moe_generate_rows(seed_x, T, H, _p(out_dev), _p(stream)))


def moe_decode_layer(shape: moe_shape_t, layer_dev: int, T: int, h_in_dev: int, h_out_dev: int,
                     ids_dev: Optional[int], w_dev: Optional[int], ws_dev: int, ws_bytes: int,
                     stream: int = 0) -> None:
    _check(lib().moe_decode_layer(ctypes.byref(shape), _p(layer_dev), T, _p(h_in_dev), _p(h_out_dev), _p(ids_dev),
                                  _p(w_dev), _p(ws_dev), ws_bytes, _p(stream)))


def moe_decode_stack(shape: moe_shape_t, layers_dev: Sequence[int], T: int, h_in_dev: int, h_out_dev: int,
                     ids_dev: Optional[int], w_dev: Optional[int], h_trace_dev: Optional[int], ws_dev: int,
                     ws_bytes: int, stream: int = 0) -> None:
    arr = (c_vp * len(layers_dev))(*[_p(p) for p in layers_dev])
    _check(lib().moe_decode_stack(ctypes.byref(shape), arr, len(layers_dev), T, _p(h_in_dev), _p(h_out_dev),
                                  _p(ids_dev), _p(w_dev), _p(h_trace_dev), _p(ws_dev), ws_bytes, _p(stream)))


def moe_decode_stack_static(shape: moe_shape_t, layers_dev: Sequence[int], T: int, h_in_dev: int, h_out_dev: int,
                            ids_dev: Optional[int], w_dev: Optional[int], h_trace_dev: Optional[int],
                            stream: int = 0) -> None:
    arr = (c_vp * len(layers_dev))(*[_p(p) for p in layers_dev])
    _check(lib().moe_decode_stack_static(ctypes.byref(shape), arr, len(layers_dev), T, _p(h_in_dev), _p(h_out_dev),
                                         _p(ids_dev), _p(w_dev), _p(h_trace_dev), _p(stream)))


def moe_stack_init(shape: moe_shape_t, layers_dev: Sequence[int], t_max: int, flags: int, ws_dev: int,
                   ws_bytes: int, stream: int = 0) -> moe_stack_t:
    st = moe_stack_t()
    arr = (c_vp * len(layers_dev))(*[_p(p) for p in layers_dev])
    _check(lib().moe_stack_init(ctypes.byref(st), ctypes.byref(shape), arr, len(layers_dev), t_max, flags, _p(ws_dev),
                                ws_bytes, _p(stream)))
    return st


def moe_stack_decode(st: moe_stack_t, T: int, h_in_dev: int, h_out_dev: int, ids_dev: Optional[int],
                     w_dev: Optional[int], h_trace_dev: Optional[int], stream: int = 0) -> None:
    _check(lib().moe_stack_decode(ctypes.byref(st), T, _p(h_in_dev), _p(h_out_dev), _p(ids_dev), _p(w_dev),
                                  _p(h_trace_dev), _p(stream)))


def moe_stack_status(shape: moe_shape_t, T: int, ws_dev: int, stream: int = 0) -> int:
    v = ctypes.c_uint32(0)
    _check(lib().moe_stack_status(ctypes.byref(shape), T, _p(ws_dev), ctypes.byref(v), _p(stream)))
    return v.value


def moe_gemv(bits: int, cols: int, T: int, x_dev: int, mats: Sequence, stream: int = 0) -> None:
    """mats: sequence of (w_dev, rows, y_dev) device addresses / row counts."""
    arr = (moe_gemv_mat_t * max(1, len(mats)))()
    for i, (w, r, y) in enumerate(mats):
        arr[i] = moe_gemv_mat_t(_p(w), r, 0, _p(y))
    _check(lib().moe_gemv(bits, cols, T, _p(x_dev), arr, len(mats), _p(stream)))


def moe_generate_matrix(bits: int, rows: int, cols: int, seed: int, layer: int, tensor: int, dst_dev: int,
                        stream: int = 0) -> None:
    _check(lib().moe_generate_matrix(bits, rows, cols, seed, layer, tensor, _p(dst_dev), _p(stream)))


def moe_gqa_workspace_bytes(shape: moe_attn_shape_t, T: int) -> int:
    return _check(lib().moe_gqa_workspace_bytes(ctypes.byref(shape), T))


def moe_gqa_decode(shape: moe_attn_shape_t, T: int, p0: int, q_dev: int, k_dev: int, v_dev: int, o_dev: int,
                   ws_dev: int, ws_bytes: int, stream: int = 0) -> None:
    _check(lib().moe_gqa_decode(ctypes.byref(shape), T, p0, _p(q_dev), _p(k_dev), _p(v_dev), _p(o_dev), _p(ws_dev),
                                ws_bytes, _p(stream)))


def moe_gdn_step(shape: moe_gdn_shape_t, T: int, state_dev: int, q_dev: int, k_dev: int, v_dev: int,
                 alpha_dev: int, beta_dev: int, o_dev: int, stream: int = 0) -> None:
    _check(lib().moe_gdn_step(ctypes.byref(shape), T, _p(state_dev), _p(q_dev), _p(k_dev), _p(v_dev), _p(alpha_dev),
                              _p(beta_dev), _p(o_dev), _p(stream)))


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_version() -> str:
    return lib().moe_version().decode()
