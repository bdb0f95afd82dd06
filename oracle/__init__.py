"""fp64 CPU oracle for jagged attention (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does; the two
share no code.  The arithmetic lives in ``jfa_oracle.c`` (plain C, fp64); this
module only marshals numpy arrays into it.

Conventions (see ``jfa_oracle.c`` for the page citations):
  q [Tq, H, d], k/v [Tkv, H, d], o like q, lse [H, Tq]; offsets int64 [B+1].
  mode: "softmax" | "silu" | "gelu"; bias_kind: "none" | "relpos" | "dense".
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "jfa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libjfa_oracle.so")

MODES = {"softmax": 0, "silu": 1, "gelu": 2}
BIAS = {"none": 0, "relpos": 1, "dense": 2}


def build(force: bool = False) -> str:
    """Compiles the oracle with gcc (plain -O2, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-ffp-contract=off",
                               "-fno-fast-math", "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp,
                               "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("scale", ctypes.c_double),
                ("normalize", ctypes.c_int32), ("bias_kind", ctypes.c_int32),
                ("num_buckets", ctypes.c_int32), ("block", ctypes.c_int32),
                ("window", ctypes.c_int32)]


class _SchedParams(ctypes.Structure):
    _fields_ = [("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("slots", ctypes.c_int32),
                ("bq_bm", ctypes.c_int32), ("bq_bn", ctypes.c_int32),
                ("bk_bn", ctypes.c_int32), ("bk_bm", ctypes.c_int32),
                ("fuse", ctypes.c_int32), ("window", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        _lib.ora_offsets.argtypes = [P, ctypes.c_int32, P]
        _lib.ora_bias_offsets.argtypes = [P, P, ctypes.c_int32, P]
        _lib.ora_block_offsets.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int64]
        _lib.ora_block_offsets.restype = ctypes.c_int64
        _lib.ora_relpos_bucket.argtypes = [ctypes.c_int64, ctypes.c_int32]
        _lib.ora_relpos_bucket.restype = ctypes.c_int
        _lib.ora_forward.argtypes = [P] * 10
        _lib.ora_backward.argtypes = [P] * 12
        _lib.ora_bias_grad.argtypes = [P] * 10
        _lib.ora_abs_terms.argtypes = [P] * 13
        _lib.ora_schedule.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P,
                                      P, P, P, P, P, ctypes.c_int64, P]
        _lib.ora_e4m3_decode.argtypes = [ctypes.c_int]
        _lib.ora_e4m3_decode.restype = ctypes.c_double
        _lib.ora_mxfp8_quantize.argtypes = [P, ctypes.c_int64, ctypes.c_int32, P, P]
        _lib.ora_mxfp8_dequantize.argtypes = [P, P, ctypes.c_int64, ctypes.c_int32, P]
        _lib.ora_set_threads.argtypes = [ctypes.c_int]
        _lib.ora_max_threads.restype = ctypes.c_int
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):           # a CPU torch tensor
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def set_threads(n: int) -> None:
    lib().ora_set_threads(int(n))


def max_threads() -> int:
    return int(lib().ora_max_threads())


# ------------------------------------------------------------------ offsets

def offsets(lengths) -> np.ndarray:
    """Exclusive prefix sum of per-sample lengths (int64 [B+1])."""
    ln = np.ascontiguousarray(lengths, dtype=np.int32)
    out = np.zeros(ln.shape[0] + 1, dtype=np.int64)
    if lib().ora_offsets(_ptr(ln), ln.shape[0], _ptr(out)) != 0:
        raise ValueError("negative length")
    return out


def bias_offsets(q_lens, kv_lens) -> np.ndarray:
    """Start of each sample's block in a dense jagged bias, in units of H elements."""
    a = np.ascontiguousarray(q_lens, dtype=np.int32)
    b = np.ascontiguousarray(kv_lens, dtype=np.int32)
    out = np.zeros(a.shape[0] + 1, dtype=np.int64)
    if lib().ora_bias_offsets(_ptr(a), _ptr(b), a.shape[0], _ptr(out)) != 0:
        raise ValueError("negative length")
    return out


def block_batch_bound(batch: int, total_rows: int, block: int) -> int:
    """Refined batch size that always holds the blocks: sum_b ceil(n_b / W) <= B + T // W."""
    return int(batch) + int(total_rows) // int(block)


def block_offsets(offsets_, block: int, out_batch: Optional[int] = None) -> np.ndarray:
    """BlockAttention's refined offsets (int64 [out_batch + 1]); see ``ora_block_offsets``."""
    off = np.ascontiguousarray(offsets_, dtype=np.int64)
    B = off.shape[0] - 1
    if out_batch is None:
        out_batch = block_batch_bound(B, int(off[-1]), block)
    out = np.zeros(out_batch + 1, dtype=np.int64)
    if lib().ora_block_offsets(_ptr(off), B, int(block), _ptr(out), int(out_batch)) < 0:
        raise ValueError("blocks exceed out_batch, or block < 1")
    return out


def relpos_bucket(delta: int, num_buckets: int = 64) -> int:
    return int(lib().ora_relpos_bucket(int(delta), int(num_buckets)))


# ------------------------------------------------------------ attention

def _problem(B, H, d, mode, causal, scale, normalize, bias_kind, num_buckets, block=0,
             window=0):
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if normalize is None:
        normalize = mode != "softmax"
    assert int(window) >= 0
    return _Problem(B, H, d, MODES[mode], int(bool(causal)), float(scale), int(bool(normalize)),
                    BIAS[bias_kind], int(num_buckets), int(block), int(window))


def _check_block(block, q_lens, kv_lens, bias_kind):
    if block:
        # BlockAttention is self-attention over one sequence: blocks are the same rows on both
        # sides; a dense bias is defined on the refined batch, not here
        assert block > 0 and bias_kind != "dense"
        assert np.array_equal(np.asarray(q_lens), np.asarray(kv_lens))


def forward(q, k, v, q_lens, kv_lens, *, mode="softmax", causal=False, bias=None,
            bias_kind="none", num_buckets=64, scale=None, normalize=None, block=0, window=0):
    """Returns (o [Tq,H,d] fp64, lse [H,Tq] fp64 or None for GDPA).  block > 0: BlockAttention
    with blocks of that many rows; window > 0: sliding window, key j visible to query i only
    when |i + (kv_len - q_len) - j| < window (and j <= i + kv_len - q_len when causal)."""
    _check_block(block, q_lens, kv_lens, bias_kind)
    q, k, v = _f64(q), _f64(k), _f64(v)
    Tq, H, d = q.shape
    qo, ko = offsets(q_lens), offsets(kv_lens)
    B = qo.shape[0] - 1
    assert qo[-1] == Tq and ko[-1] == k.shape[0] and k.shape == v.shape
    bo = bias_offsets(q_lens, kv_lens)
    bias64 = _f64(bias) if bias is not None else None
    if bias_kind != "none":
        assert bias64 is not None
    p = _problem(B, H, d, mode, causal, scale, normalize, bias_kind, num_buckets, block,
                 window)
    o = np.zeros_like(q)
    lse = np.full((H, Tq), np.nan) if mode == "softmax" else None
    lib().ora_forward(ctypes.byref(p), _ptr(qo), _ptr(ko), _ptr(q), _ptr(k), _ptr(v),
                      _ptr(bias64), _ptr(bo), _ptr(o), _ptr(lse))
    return o, lse


def backward(q, k, v, dout, q_lens, kv_lens, *, mode="softmax", causal=False, bias=None,
             bias_kind="none", num_buckets=64, scale=None, normalize=None, block=0, window=0):
    """Returns (dq, dk, dv) in fp64: the gradients of <O, dout>."""
    _check_block(block, q_lens, kv_lens, bias_kind)
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    Tq, H, d = q.shape
    qo, ko = offsets(q_lens), offsets(kv_lens)
    B = qo.shape[0] - 1
    bo = bias_offsets(q_lens, kv_lens)
    bias64 = _f64(bias) if bias is not None else None
    p = _problem(B, H, d, mode, causal, scale, normalize, bias_kind, num_buckets, block,
                 window)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    lib().ora_backward(ctypes.byref(p), _ptr(qo), _ptr(ko), _ptr(q), _ptr(k), _ptr(v),
                       _ptr(bias64), _ptr(bo), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv))
    return dq, dk, dv


def bias_grad(q, k, v, dout, q_lens, kv_lens, *, mode="softmax", causal=False, bias=None,
              bias_kind="relpos", num_buckets=64, scale=None, normalize=None, block=0, window=0):
    """Gradient of <O, dout> with respect to the bias (fp64): the relative-position table
    [H][num_buckets], or a dense bias in its own layout."""
    assert bias_kind in ("relpos", "dense") and bias is not None
    _check_block(block, q_lens, kv_lens, bias_kind)
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    Tq, H, d = q.shape
    qo, ko = offsets(q_lens), offsets(kv_lens)
    B = qo.shape[0] - 1
    bo = bias_offsets(q_lens, kv_lens)
    bias64 = _f64(bias)
    p = _problem(B, H, d, mode, causal, scale, normalize, bias_kind, num_buckets, block,
                 window)
    db = np.zeros_like(bias64)
    lib().ora_bias_grad(ctypes.byref(p), _ptr(qo), _ptr(ko), _ptr(q), _ptr(k), _ptr(v),
                        _ptr(bias64), _ptr(bo), _ptr(dout), _ptr(db))
    return db


def abs_terms(q, k, v, dout, q_lens, kv_lens, *, mode="softmax", causal=False, bias=None,
              bias_kind="none", num_buckets=64, scale=None, normalize=None, block=0, window=0):
    """Absolute-value contractions (fp64) behind each output element: dict with "O" = sum_j
    |P_ij||V_j|, "dV" = sum_i |P_ij||dO_i|, "dQ" = scale sum_j |dS_ij||K_j|, "dK" = scale
    sum_i |dS_ij||Q_i| (GDPA's P includes its weight w).  Rounding P or dS to a format with
    relative error u moves each output by at most u times its term (see ``ora_abs_terms``).
    dout None: only "O"."""
    _check_block(block, q_lens, kv_lens, bias_kind)
    q, k, v = _f64(q), _f64(k), _f64(v)
    dout = None if dout is None else _f64(dout)
    Tq, H, d = q.shape
    qo, ko = offsets(q_lens), offsets(kv_lens)
    B = qo.shape[0] - 1
    bo = bias_offsets(q_lens, kv_lens)
    bias64 = _f64(bias) if bias is not None else None
    p = _problem(B, H, d, mode, causal, scale, normalize, bias_kind, num_buckets, block,
                 window)
    c_o = np.zeros_like(q)
    c_dq, c_dk, c_dv = (np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)) \
        if dout is not None else (None, None, None)
    lib().ora_abs_terms(ctypes.byref(p), _ptr(qo), _ptr(ko), _ptr(q), _ptr(k), _ptr(v),
                        _ptr(bias64), _ptr(bo), _ptr(dout), _ptr(c_o), _ptr(c_dq), _ptr(c_dk),
                        _ptr(c_dv))
    out = {"O": c_o}
    if dout is not None:
        out.update(dQ=c_dq, dK=c_dk, dV=c_dv)
    return out


def case_abs_terms(case, **kw):
    return abs_terms(case.q, case.k, case.v, case.dout, case.q_lens, case.kv_lens,
                     mode=case.mode, causal=case.causal, bias=case.bias,
                     bias_kind=case.bias_kind, num_buckets=case.num_buckets, **kw)


def case_forward(case, **kw):
    """Oracle forward on a ``jfa_synth.Case`` (values widened exactly to fp64)."""
    return forward(case.q, case.k, case.v, case.q_lens, case.kv_lens, mode=case.mode,
                   causal=case.causal, bias=case.bias, bias_kind=case.bias_kind,
                   num_buckets=case.num_buckets, **kw)


def case_backward(case, **kw):
    return backward(case.q, case.k, case.v, case.dout, case.q_lens, case.kv_lens,
                    mode=case.mode, causal=case.causal, bias=case.bias,
                    bias_kind=case.bias_kind, num_buckets=case.num_buckets, **kw)


# ------------------------------------------------------------- tile lists

def schedule(q_offsets, kv_offsets, heads: int, causal: bool, *, bm: int, bn: int, slots: int,
             bq_bm: int, bq_bn: int, bk_bn: int, bk_bm: int, fuse: int = 3,
             window: int = 0) -> dict:
    """Forward / combine / backward tile lists (see ``ora_schedule`` in the C source).

    fuse: single-pass backward classes, bit 0 for samples with one query tile, bit 1 for
    samples with one key tile (True means both).  window: the attention's sliding window
    (0 = none); tiles then cover only the steps some of their rows can see."""
    qo = np.ascontiguousarray(q_offsets, dtype=np.int64)
    ko = np.ascontiguousarray(kv_offsets, dtype=np.int64)
    B = qo.shape[0] - 1
    n = np.diff(qo)
    m = np.diff(ko)
    cap = int(np.sum((n + 1)) + np.sum(m + 1) + 64 + 2 * max(slots, 0) + 16)
    cap += int(np.sum(-(-np.maximum(m, 1) // min(bn, bq_bn, bk_bn)) * (-(-np.maximum(n, 1) // min(bm, bq_bm)))))
    fwd = np.zeros((cap, 4), np.int32)
    fslot = np.zeros(cap, np.int32)
    comb = np.zeros((cap, 4), np.int32)
    bq = np.zeros((cap, 4), np.int32)
    bk = np.zeros((cap, 4), np.int32)
    counts = np.zeros(5, np.int64)
    fuse = 3 if fuse is True else int(fuse)
    sp = _SchedParams(bm, bn, slots, bq_bm, bq_bn, bk_bn, bk_bm, fuse, int(window))
    rc = lib().ora_schedule(_ptr(qo), _ptr(ko), B, heads, int(bool(causal)), ctypes.byref(sp),
                            _ptr(fwd), _ptr(fslot), _ptr(comb), _ptr(bq), _ptr(bk), cap,
                            _ptr(counts))
    if rc == -1:
        raise ValueError("malformed offsets")
    if rc != 0:
        raise RuntimeError(f"ora_schedule failed ({rc})")
    nf, nc, nq, nk, C = (int(x) for x in counts)
    return dict(fwd=fwd[:nf].copy(), fwd_slot=fslot[:nf].copy(), combine=comb[:nc].copy(),
                bwd_q=bq[:nq].copy(), bwd_kv=bk[:nk].copy(), split_threshold=C)


# ------------------------------------------------------------------ MXFP8

def rmsnorm(x, weight=None, n=None, eps=1e-6):
    """RMS normalisation in fp64 over groups of n consecutive elements (default: the last
    dimension): y = x / sqrt(mean(x^2) + eps) * weight.  The normalisation into which the
    quantisation is fused ("Meta GEM Training Efficiency: ...", section "Bottleneck move 2"; the
    pages do not name the normalisation, RMS normalisation with a per-channel gain is the
    reading taken here)."""
    x = _f64(x)
    n = x.shape[-1] if n is None else int(n)
    g = x.reshape(-1, n)
    y = g / np.sqrt(np.mean(g * g, axis=1, keepdims=True) + float(eps))
    if weight is not None:
        y = y * _f64(weight).reshape(1, n)
    return y.reshape(x.shape)


def e4m3_decode(code: int) -> float:
    return float(lib().ora_e4m3_decode(int(code)))


def mxfp8_quantize(x):
    """x [..., d] -> (codes uint8 [..., d], scales uint8 [..., d/32])."""
    x = _f64(x)
    d = x.shape[-1]
    rows = int(np.prod(x.shape[:-1])) if x.ndim > 1 else 1
    codes = np.zeros(x.shape, np.uint8)
    scales = np.zeros(x.shape[:-1] + (d // 32,), np.uint8)
    if lib().ora_mxfp8_quantize(_ptr(x), rows, d, _ptr(codes), _ptr(scales)) != 0:
        raise ValueError("d must be a multiple of 32")
    return codes, scales


def mxfp8_dequantize(codes, scales) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    d = codes.shape[-1]
    rows = int(np.prod(codes.shape[:-1])) if codes.ndim > 1 else 1
    out = np.zeros(codes.shape, np.float64)
    lib().ora_mxfp8_dequantize(_ptr(codes), _ptr(scales), rows, d, _ptr(out))
    return out
