"""ctypes binding of libjfa.so: one Python function per C entry point, same names.

Argument marshalling only: torch tensors become device pointers, the current HIP
stream becomes the stream argument.  Every computation happens in the library's
HIP kernels; there is no fallback.  If libjfa.so is missing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libjfa.so")

JFA_OK = 0
JFA_ERR_INVALID_ARG = -1
JFA_ERR_UNSUPPORTED = -2
JFA_ERR_WORKSPACE = -3
JFA_ERR_LAUNCH = -4
JFA_ERR_DEVICE_DATA = -5

NOALLOC_SCRATCH_BYTES = 64 << 20     # JFA_NOALLOC_SCRATCH_BYTES

MODES = {"softmax": 0, "silu": 1, "gelu": 2}
DTYPES = {"f32": 0, "bf16": 1, "mxfp8": 2}
BIAS_KINDS = {"none": 0, "relpos": 1, "dense": 2}

# every symbol include/jfa.h declares
EXPORTS = ("jfa_workspace_bytes", "jfa_forward", "jfa_forward_noalloc", "jfa_backward",
           "jfa_backward_mxfp8", "jfa_backward_dbias",
           "jfa_tile_config",
           "jfa_build_schedule", "jfa_lengths_to_offsets", "jfa_block_offsets",
           "jfa_quantize_mxfp8", "jfa_quantize_mxfp8_batch", "jfa_rmsnorm_quantize_mxfp8",
           "jfa_read_device_status", "jfa_status_string", "jfa_set_kernel_timing",
           "jfa_kernel_timing", "jfa_kernel_timing_reset")


class JfaProblem(ctypes.Structure):
    """Mirror of jfa_problem (include/jfa.h)."""
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("total_q", ctypes.c_int64),
                ("total_kv", ctypes.c_int64), ("mode", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("qk_scale", ctypes.c_float), ("kv_len_normalize", ctypes.c_int32),
                ("bias_kind", ctypes.c_int32), ("num_buckets", ctypes.c_int32),
                ("split_slots", ctypes.c_int32), ("bwd_fuse", ctypes.c_int32),
                ("window", ctypes.c_int32)]


class JfaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Loads libjfa.so (built in-tree by jagged_attention_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m jagged_attention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    PP = ctypes.POINTER(JfaProblem)
    lib.jfa_workspace_bytes.argtypes = [PP, ctypes.c_int]
    lib.jfa_workspace_bytes.restype = SZ
    lib.jfa_forward.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.jfa_forward.restype = ctypes.c_int
    lib.jfa_forward_noalloc.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.jfa_forward_noalloc.restype = ctypes.c_int
    lib.jfa_backward.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.jfa_backward.restype = ctypes.c_int
    lib.jfa_backward_mxfp8.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                       SZ, P]
    lib.jfa_backward_mxfp8.restype = ctypes.c_int
    lib.jfa_backward_dbias.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.jfa_backward_dbias.restype = ctypes.c_int
    lib.jfa_tile_config.argtypes = [PP, P]
    lib.jfa_tile_config.restype = ctypes.c_int
    lib.jfa_build_schedule.argtypes = [PP, P, P, P, P, P, P, P, P, I64, P, SZ, P]
    lib.jfa_build_schedule.restype = ctypes.c_int
    lib.jfa_lengths_to_offsets.argtypes = [P, I32, P, P, P, P, P]
    lib.jfa_lengths_to_offsets.restype = ctypes.c_int
    lib.jfa_block_offsets.argtypes = [P, I32, I32, P, I32, P, P]
    lib.jfa_block_offsets.restype = ctypes.c_int
    lib.jfa_quantize_mxfp8.argtypes = [P, I64, I32, P, P, P]
    lib.jfa_quantize_mxfp8.restype = ctypes.c_int
    lib.jfa_quantize_mxfp8_batch.argtypes = [I32, P, P, I32, P, P, P]
    lib.jfa_quantize_mxfp8_batch.restype = ctypes.c_int
    lib.jfa_rmsnorm_quantize_mxfp8.argtypes = [P, P, I64, I32, ctypes.c_float, P, P, P]
    lib.jfa_rmsnorm_quantize_mxfp8.restype = ctypes.c_int
    lib.jfa_read_device_status.argtypes = [P, P, ctypes.POINTER(I32)]
    lib.jfa_read_device_status.restype = ctypes.c_int
    lib.jfa_status_string.argtypes = [ctypes.c_int]
    lib.jfa_status_string.restype = ctypes.c_char_p
    lib.jfa_set_kernel_timing.argtypes = [ctypes.c_int]
    lib.jfa_set_kernel_timing.restype = None
    lib.jfa_kernel_timing.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(I64)]
    lib.jfa_kernel_timing.restype = ctypes.c_int
    lib.jfa_kernel_timing_reset.argtypes = []
    lib.jfa_kernel_timing_reset.restype = None
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().jfa_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != JFA_OK:
        raise JfaError(fn, status)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


# ------------------------------------------------------- one per entry point

def jfa_workspace_bytes(problem: JfaProblem, backward: int) -> int:
    """backward: 0 forward, 1 (or True) backward, 2 backward with the bias gradient."""
    return int(load().jfa_workspace_bytes(ctypes.byref(problem), int(backward)))


def jfa_forward(problem, q, k, v, q_scale, k_scale, v_scale, q_offsets, kv_offsets, bias, o, lse,
                workspace, workspace_bytes: int, stream=None) -> None:
    st = load().jfa_forward(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale),
                            _ptr(k_scale), _ptr(v_scale), _ptr(q_offsets), _ptr(kv_offsets),
                            _ptr(bias), _ptr(o), _ptr(lse), _ptr(workspace), workspace_bytes,
                            _stream(stream))
    _check("jfa_forward", st)


def jfa_forward_noalloc(problem, q, k, v, q_scale, k_scale, v_scale, q_offsets, kv_offsets, bias,
                        o, lse, stream=None) -> None:
    st = load().jfa_forward_noalloc(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
                                    _ptr(q_offsets), _ptr(kv_offsets), _ptr(bias), _ptr(o),
                                    _ptr(lse), _stream(stream))
    _check("jfa_forward_noalloc", st)


def jfa_backward(problem, q, k, v, o, lse, dout, q_offsets, kv_offsets, bias, dq, dk, dv,
                 workspace, workspace_bytes: int, stream=None) -> None:
    st = load().jfa_backward(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                             _ptr(dout), _ptr(q_offsets), _ptr(kv_offsets), _ptr(bias), _ptr(dq),
                             _ptr(dk), _ptr(dv), _ptr(workspace), workspace_bytes, _stream(stream))
    _check("jfa_backward", st)


def jfa_backward_mxfp8(problem, q, k, v, q_scale, k_scale, v_scale, o, lse, dout, dout_scale,
                       q_offsets, kv_offsets, bias, dq, dk, dv, workspace, workspace_bytes: int,
                       stream=None) -> None:
    st = load().jfa_backward_mxfp8(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), _ptr(o),
                                   _ptr(lse), _ptr(dout), _ptr(dout_scale), _ptr(q_offsets),
                                   _ptr(kv_offsets), _ptr(bias), _ptr(dq), _ptr(dk), _ptr(dv),
                                   _ptr(workspace), workspace_bytes, _stream(stream))
    _check("jfa_backward_mxfp8", st)


def jfa_backward_dbias(problem, q, k, v, o, lse, dout, q_offsets, kv_offsets, bias, dq, dk, dv,
                       dbias, workspace, workspace_bytes: int, stream=None) -> None:
    st = load().jfa_backward_dbias(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                   _ptr(lse), _ptr(dout), _ptr(q_offsets), _ptr(kv_offsets),
                                   _ptr(bias), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias),
                                   _ptr(workspace), workspace_bytes, _stream(stream))
    _check("jfa_backward_dbias", st)


def jfa_tile_config(problem: JfaProblem) -> dict:
    out = (ctypes.c_int32 * 8)()
    _check("jfa_tile_config", load().jfa_tile_config(ctypes.byref(problem), out))
    keys = ("bm", "bn", "slots", "bq_bm", "bq_bn", "bk_bn", "bk_bm", "fuse")
    return dict(zip(keys, list(out)))


def jfa_build_schedule(problem, q_offsets, kv_offsets, fwd, fwd_slot, comb, bwd_q, bwd_kv, counts,
                       capacity: int, workspace, workspace_bytes: int, stream=None) -> None:
    st = load().jfa_build_schedule(ctypes.byref(problem), _ptr(q_offsets), _ptr(kv_offsets),
                                   _ptr(fwd), _ptr(fwd_slot), _ptr(comb), _ptr(bwd_q),
                                   _ptr(bwd_kv), _ptr(counts), int(capacity), _ptr(workspace),
                                   workspace_bytes, _stream(stream))
    _check("jfa_build_schedule", st)


def jfa_lengths_to_offsets(lengths, batch: int, offsets, bias_offsets=None, kv_lengths=None,
                           status=None, stream=None) -> None:
    st = load().jfa_lengths_to_offsets(_ptr(lengths), int(batch), _ptr(offsets),
                                       _ptr(bias_offsets), _ptr(kv_lengths), _ptr(status),
                                       _stream(stream))
    _check("jfa_lengths_to_offsets", st)


def jfa_block_offsets(offsets, batch: int, block: int, block_offsets, out_batch: int,
                      status=None, stream=None) -> None:
    st = load().jfa_block_offsets(_ptr(offsets), int(batch), int(block), _ptr(block_offsets),
                                  int(out_batch), _ptr(status), _stream(stream))
    _check("jfa_block_offsets", st)


def jfa_quantize_mxfp8(x, rows: int, d: int, codes, scales, stream=None) -> None:
    st = load().jfa_quantize_mxfp8(_ptr(x), int(rows), int(d), _ptr(codes), _ptr(scales),
                                   _stream(stream))
    _check("jfa_quantize_mxfp8", st)


def jfa_quantize_mxfp8_batch(xs, rows, d: int, codes, scales, stream=None) -> None:
    """xs, codes, scales: lists of device tensors (1 to 4); rows: their row counts."""
    n = len(xs)
    arr = lambda ts: (ctypes.c_void_p * n)(*[_ptr(t) for t in ts])
    rws = (ctypes.c_int64 * n)(*[int(r) for r in rows])
    st = load().jfa_quantize_mxfp8_batch(n, arr(xs), rws, int(d), arr(codes), arr(scales),
                                         _stream(stream))
    _check("jfa_quantize_mxfp8_batch", st)


def jfa_rmsnorm_quantize_mxfp8(x, weight, groups: int, n: int, eps: float, codes, scales,
                               stream=None) -> None:
    st = load().jfa_rmsnorm_quantize_mxfp8(_ptr(x), _ptr(weight), int(groups), int(n),
                                           float(eps), _ptr(codes), _ptr(scales),
                                           _stream(stream))
    _check("jfa_rmsnorm_quantize_mxfp8", st)


def jfa_read_device_status(workspace, stream=None) -> int:
    out = ctypes.c_int32(0)
    _check("jfa_read_device_status",
           load().jfa_read_device_status(_ptr(workspace), _stream(stream), ctypes.byref(out)))
    return int(out.value)


def jfa_set_kernel_timing(enable: bool) -> None:
    load().jfa_set_kernel_timing(int(bool(enable)))


def jfa_kernel_timing(name_prefix: str = "") -> tuple:
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check("jfa_kernel_timing", load().jfa_kernel_timing(name_prefix.encode(), ctypes.byref(ms),
                                                         ctypes.byref(n)))
    return float(ms.value), int(n.value)


def jfa_kernel_timing_reset() -> None:
    load().jfa_kernel_timing_reset()
