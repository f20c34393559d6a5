"""Python binding of libhq.so, the MI355X fused-dequantization quantized GEMM (include/hq.h).

Argument marshalling only: every function forwards to the C entry point of the same name.
Device buffers are anything with a ``data_ptr()`` (PyTorch tensors on the GPU); host buffers
for the prepack are numpy arrays. A non-OK status raises :class:`HQError` carrying the
library's message. The library must be built (``python -m quantized_gemm_prepacked_amd.build``
or ``__graft_entry__.build()``); importing without it raises ImportError -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
# PyTorch's HIP runtime must be the one loaded before libhq.so: the library then binds to that
# same runtime (device memory and streams come from PyTorch).
import torch  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with quantized_gemm_prepacked_amd/build.py")

_lib = ctypes.CDLL(LIB_PATH)

# ---- enums (hq.h) -----------------------------------------------------------------------------
HQ_OK, HQ_ERR_INVALID_ARGUMENT, HQ_ERR_UNSUPPORTED, HQ_ERR_WORKSPACE, HQ_ERR_HIP = range(5)
HQ_W_INT4_SYM, HQ_W_UINT4_ASYM, HQ_W_INT8_SYM, HQ_W_FP4_E2M1, HQ_W_FP8_E4M3, HQ_W_UINT2_ASYM, HQ_W_UINT3_ASYM = range(7)
HQ_SCALE_BF16, HQ_SCALE_FP32, HQ_SCALE_E8M0 = range(3)
HQ_ACT_BF16, HQ_ACT_INT8_PER_TOKEN, HQ_ACT_FP8E4M3_PER_TOKEN, HQ_ACT_MXFP4, HQ_ACT_MXFP8, HQ_ACT_FP8E4M3_BLOCK128 = range(6)
HQ_OUT_BF16, HQ_OUT_INT32_ACC = range(2)

EXPORTED = (
    "hq_prepacked_bytes", "hq_prepack_weights", "hq_gemm_workspace_bytes", "hq_gemm", "hq_gemm_noalloc",
    "hq_moe_align_capacity", "hq_moe_align_workspace_bytes", "hq_moe_align", "hq_moe_block_m",
    "hq_moe_gemm_workspace_bytes", "hq_moe_grouped_gemm", "hq_quantize_activations",
    "hq_moe_silu_mul", "hq_moe_silu_mul_quantize", "hq_moe_combine", "hq_grouped_gemm_workspace_bytes",
    "hq_grouped_gemm",
    "hq_load_tuning_table", "hq_gemm_plan", "hq_kernel_config_count",
    "hq_last_error", "hq_version",
)


class hq_quant_desc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("weight_fmt", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("scale_dtype", ctypes.c_int32),
        ("has_zero_point", ctypes.c_int32),
        ("act_fmt", ctypes.c_int32),
        ("out_fmt", ctypes.c_int32),
        ("compute_flags", ctypes.c_int32),
    ]


HQ_COMPUTE_BATCH_INVARIANT = 1
HQ_COMPUTE_STREAM_K = 2


def make_desc(weight_fmt, group_size, scale_dtype, has_zero_point, act_fmt, out_fmt=HQ_OUT_BF16,
              compute_flags=0):
    return hq_quant_desc(ctypes.sizeof(hq_quant_desc), weight_fmt, group_size, scale_dtype,
                         has_zero_point, act_fmt, out_fmt, compute_flags)


def with_flags(desc, compute_flags):
    """A copy of `desc` with its compute flags set (e.g. HQ_COMPUTE_BATCH_INVARIANT)."""
    return make_desc(desc.weight_fmt, desc.group_size, desc.scale_dtype, desc.has_zero_point,
                     desc.act_fmt, desc.out_fmt, compute_flags)


# The four supported combinations (plus the W8A8 raw-accumulator test mode).
DESC_W4A16_SYM = make_desc(HQ_W_INT4_SYM, 128, HQ_SCALE_BF16, 0, HQ_ACT_BF16)
DESC_W4A16_ASYM = make_desc(HQ_W_UINT4_ASYM, 128, HQ_SCALE_BF16, 1, HQ_ACT_BF16)
DESC_W8A8 = make_desc(HQ_W_INT8_SYM, 0, HQ_SCALE_FP32, 0, HQ_ACT_INT8_PER_TOKEN)
DESC_W8A8_I32 = make_desc(HQ_W_INT8_SYM, 0, HQ_SCALE_FP32, 0, HQ_ACT_INT8_PER_TOKEN, HQ_OUT_INT32_ACC)
DESC_W4A8_MXFP4 = make_desc(HQ_W_FP4_E2M1, 32, HQ_SCALE_E8M0, 0, HQ_ACT_FP8E4M3_PER_TOKEN)
DESC_W4A4_MXFP4 = make_desc(HQ_W_FP4_E2M1, 32, HQ_SCALE_E8M0, 0, HQ_ACT_MXFP4)
DESC_W4A8_MXFP8 = make_desc(HQ_W_FP4_E2M1, 32, HQ_SCALE_E8M0, 0, HQ_ACT_MXFP8)
DESC_W4A16_MXFP4 = make_desc(HQ_W_FP4_E2M1, 32, HQ_SCALE_E8M0, 0, HQ_ACT_BF16)
DESC_W8A8_FP8_BLOCK = make_desc(HQ_W_FP8_E4M3, 128, HQ_SCALE_FP32, 0, HQ_ACT_FP8E4M3_BLOCK128)
DESC_W8A16_INT8 = make_desc(HQ_W_INT8_SYM, 0, HQ_SCALE_FP32, 0, HQ_ACT_BF16)
DESC_W8A16_FP8 = make_desc(HQ_W_FP8_E4M3, 0, HQ_SCALE_FP32, 0, HQ_ACT_BF16)
DESC_W2A16_ASYM = make_desc(HQ_W_UINT2_ASYM, 128, HQ_SCALE_BF16, 1, HQ_ACT_BF16)
DESC_W3A16_ASYM = make_desc(HQ_W_UINT3_ASYM, 128, HQ_SCALE_BF16, 1, HQ_ACT_BF16)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_D = ctypes.POINTER(hq_quant_desc)


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_c = {
    "hq_prepacked_bytes": _sig("hq_prepacked_bytes", _SZ, _D, _I64, _I64, _I64),
    "hq_prepack_weights": _sig("hq_prepack_weights", ctypes.c_int, _D, _I64, _I64, _I64, _P, _P, _P, _P, _SZ),
    "hq_gemm_workspace_bytes": _sig("hq_gemm_workspace_bytes", _SZ, _D, _I64, _I64, _I64),
    "hq_gemm": _sig("hq_gemm", ctypes.c_int, _D, _I64, _I64, _I64, _P, _P, _P, _P, _P, _SZ, _P),
    "hq_gemm_noalloc": _sig("hq_gemm_noalloc", ctypes.c_int, _D, _I64, _I64, _I64, _P, _P, _P, _P, _P),
    "hq_moe_align_capacity": _sig("hq_moe_align_capacity", _SZ, _I64, _I32, _I32, _I32),
    "hq_moe_align_workspace_bytes": _sig("hq_moe_align_workspace_bytes", _SZ, _I64, _I32, _I32, _I32),
    "hq_moe_align": _sig("hq_moe_align", ctypes.c_int, _P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P),
    "hq_moe_block_m": _sig("hq_moe_block_m", _I32, _D, _I64, _I32, _I32, _I64, _I64),
    "hq_moe_gemm_workspace_bytes": _sig("hq_moe_gemm_workspace_bytes", _SZ, _D, _I64, _I32, _I32, _I64, _I64, _I32),
    "hq_moe_grouped_gemm": _sig("hq_moe_grouped_gemm", ctypes.c_int, _D, _I64, _I32, _I32, _I64, _I64, _P, _P, _P,
                                _P, _P, _P, _I32, _P, _P, _P, _SZ, _P),
    "hq_quantize_activations": _sig("hq_quantize_activations", ctypes.c_int, _I32, _I64, _I64, _P, _P, _P, _P),
    "hq_grouped_gemm_workspace_bytes": _sig("hq_grouped_gemm_workspace_bytes", ctypes.c_size_t, _P, _I64, _I32,
                                            _I64, _I64),
    "hq_grouped_gemm": _sig("hq_grouped_gemm", ctypes.c_int, _P, _I64, _I32, _I64, _I64, _P, _P, _P, _P, _P, _P,
                            ctypes.c_size_t, _P),
    "hq_load_tuning_table": _sig("hq_load_tuning_table", ctypes.c_int, ctypes.c_char_p),
    "hq_gemm_plan": _sig("hq_gemm_plan", ctypes.c_int, _P, _I64, _I64, _I64, _P, _P, _P),
    "hq_kernel_config_count": _sig("hq_kernel_config_count", _I32, _I32),
    "hq_moe_silu_mul": _sig("hq_moe_silu_mul", ctypes.c_int, _I64, _I64, _P, _P, _P),
    "hq_moe_silu_mul_quantize": _sig("hq_moe_silu_mul_quantize", ctypes.c_int, _I32, _I64, _I64, _P, _P, _P, _P),
    "hq_moe_combine": _sig("hq_moe_combine", ctypes.c_int, _I64, _I32, _I32, _I64, _P, _P, _P, _P),
    "hq_last_error": _sig("hq_last_error", ctypes.c_char_p),
    "hq_version": _sig("hq_version", _I32),
}


class HQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"hq status {status}: {message}")
        self.status = status


def _check(status: int):
    if status != HQ_OK:
        raise HQError(status, hq_last_error())


def _ptr(x):
    """Device/host address of a tensor, numpy array or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _d(desc):
    return ctypes.byref(desc)


# ---- entry points -----------------------------------------------------------------------------
def hq_last_error() -> str:
    return _c["hq_last_error"]().decode()


def hq_version() -> int:
    return _c["hq_version"]()


def hq_prepacked_bytes(desc, E, N, K) -> int:
    return _c["hq_prepacked_bytes"](_d(desc), E, N, K)


def hq_prepack_weights(desc, E, N, K, wq: np.ndarray, scales: np.ndarray, zeros, out: np.ndarray):
    """Host prepack into ``out`` (uint8 numpy array of hq_prepacked_bytes bytes)."""
    arrs = [np.ascontiguousarray(a) for a in (wq, scales)]
    z = None if zeros is None else np.ascontiguousarray(zeros)
    _check(_c["hq_prepack_weights"](_d(desc), E, N, K, _ptr(arrs[0]), _ptr(arrs[1]), _ptr(z),
                                    _ptr(out), out.nbytes))
    return out


def hq_gemm_workspace_bytes(desc, M, N, K) -> int:
    return _c["hq_gemm_workspace_bytes"](_d(desc), M, N, K)


def hq_gemm(desc, M, N, K, a, a_scale, w_packed, y, ws=None, ws_bytes=0, stream=None):
    _check(_c["hq_gemm"](_d(desc), M, N, K, _ptr(a), _ptr(a_scale), _ptr(w_packed), _ptr(y),
                         _ptr(ws), ws_bytes, _stream(stream)))


HQ_NOALLOC_SCRATCH_BYTES = 16 << 20


def hq_gemm_noalloc(desc, M, N, K, a, a_scale, w_packed, y, stream=None):
    """hq_gemm with the library's own per-GPU scratch instead of a workspace (allocates nothing)."""
    _check(_c["hq_gemm_noalloc"](_d(desc), M, N, K, _ptr(a), _ptr(a_scale), _ptr(w_packed), _ptr(y),
                                 _stream(stream)))


def hq_moe_align_capacity(T, topk, E, block_m) -> int:
    return _c["hq_moe_align_capacity"](T, topk, E, block_m)


def hq_moe_align_workspace_bytes(T, topk, E, block_m) -> int:
    return _c["hq_moe_align_workspace_bytes"](T, topk, E, block_m)


def hq_moe_align(topk_ids, T, topk, E, block_m, sorted_ids, block_expert, expert_offsets,
                 num_padded, ws=None, ws_bytes=0, stream=None):
    _check(_c["hq_moe_align"](_ptr(topk_ids), T, topk, E, block_m, _ptr(sorted_ids),
                              _ptr(block_expert), _ptr(expert_offsets), _ptr(num_padded),
                              _ptr(ws), ws_bytes, _stream(stream)))


def hq_moe_block_m(desc, T, topk, E, N, K) -> int:
    return _c["hq_moe_block_m"](_d(desc), T, topk, E, N, K)


def hq_moe_gemm_workspace_bytes(desc, T, topk, E, N, K, block_m) -> int:
    return _c["hq_moe_gemm_workspace_bytes"](_d(desc), T, topk, E, N, K, block_m)


def hq_moe_grouped_gemm(desc, T, topk, E, N, K, a, a_scale, w_packed, sorted_ids, block_expert,
                        num_padded, block_m, topk_weights, y, ws=None, ws_bytes=0, stream=None):
    _check(_c["hq_moe_grouped_gemm"](_d(desc), T, topk, E, N, K, _ptr(a), _ptr(a_scale),
                                     _ptr(w_packed), _ptr(sorted_ids), _ptr(block_expert),
                                     _ptr(num_padded), block_m, _ptr(topk_weights), _ptr(y),
                                     _ptr(ws), ws_bytes, _stream(stream)))


def hq_grouped_gemm_workspace_bytes(desc, R, E, N, K) -> int:
    return _c["hq_grouped_gemm_workspace_bytes"](_d(desc), R, E, N, K)


def hq_grouped_gemm(desc, R, E, N, K, a, a_scale, w_packed, expert_offsets, y, ws, ws_bytes, stream=None):
    _check(_c["hq_grouped_gemm"](_d(desc), R, E, N, K, _ptr(a), _ptr(a_scale), _ptr(w_packed),
                                 _ptr(expert_offsets), _ptr(y), _ptr(ws), ws_bytes, _stream(stream)))


def hq_load_tuning_table(path):
    """Replace the process-wide tuning table with the file at `path` (None clears it)."""
    _check(_c["hq_load_tuning_table"](None if path is None else os.fsencode(path)))


def hq_gemm_plan(desc, M, N, K):
    """(kind, cfg, split) that a dense call of this shape would run."""
    k, c, s = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(_c["hq_gemm_plan"](_d(desc), M, N, K, ctypes.byref(k), ctypes.byref(c), ctypes.byref(s)))
    return k.value, c.value, s.value


def hq_kernel_config_count(kind) -> int:
    return _c["hq_kernel_config_count"](kind)


def hq_quantize_activations(act_fmt, M, K, x, xq, s_tok, stream=None):
    _check(_c["hq_quantize_activations"](act_fmt, M, K, _ptr(x), _ptr(xq), _ptr(s_tok), _stream(stream)))


def hq_moe_silu_mul(R, I, gate_up, act, stream=None):
    _check(_c["hq_moe_silu_mul"](R, I, _ptr(gate_up), _ptr(act), _stream(stream)))


def hq_moe_silu_mul_quantize(act_fmt, R, I, gate_up, act_q, act_scale, stream=None):
    _check(_c["hq_moe_silu_mul_quantize"](act_fmt, R, I, _ptr(gate_up), _ptr(act_q), _ptr(act_scale),
                                          _stream(stream)))


def hq_moe_combine(T, topk, E, N, topk_ids, y, out, stream=None):
    _check(_c["hq_moe_combine"](T, topk, E, N, _ptr(topk_ids), _ptr(y), _ptr(out), _stream(stream)))
