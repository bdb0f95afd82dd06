"""Jagged flash attention (JFA) and GDPA on AMD MI355X: Python front end of libjfa.so.

Tensors are torch tensors on the GPU; every step runs in the library's HIP kernels
(see include/jfa.h for the contract).  Layouts: q/o/dout [total_q, H, d],
k/v [total_kv, H, d], lse fp32 [H, total_q], offsets int32 [B+1].
"""
from __future__ import annotations

from typing import Optional

from . import _lib
from ._lib import (BIAS_KINDS, DTYPES, JFA_OK, MODES, JfaError, JfaProblem,  # noqa: F401
                   jfa_backward, jfa_backward_dbias, jfa_block_offsets, jfa_build_schedule, jfa_forward,
                   jfa_forward_noalloc, jfa_backward_mxfp8,
                   jfa_kernel_timing,
                   jfa_kernel_timing_reset, jfa_lengths_to_offsets, jfa_quantize_mxfp8,
                   jfa_quantize_mxfp8_batch, jfa_rmsnorm_quantize_mxfp8,
                   jfa_read_device_status, jfa_set_kernel_timing, jfa_tile_config,
                   jfa_workspace_bytes, load, status_string)

jfa_status_string = status_string

__all__ = ["make_problem", "forward", "backward", "backward_mxfp8", "backward_dbias",
           "lengths_to_offsets",
           "bias_offsets",
           "block_offsets",
           "quantize_mxfp8", "rmsnorm_quantize_mxfp8",
           "build_schedule", "JaggedAttention", "load"]


def make_problem(batch: int, heads: int, head_dim: int, total_q: int, total_kv: int, *,
                 mode: str = "softmax", dtype: str = "bf16", causal: bool = False,
                 qk_scale: float = 0.0, kv_len_normalize: int = -1, bias_kind: str = "none",
                 num_buckets: int = 64, split_slots: int = 0, bwd_fuse: int = -1,
                 window: int = 0) -> JfaProblem:
    return JfaProblem(batch=batch, heads=heads, head_dim=head_dim, total_q=total_q,
                      total_kv=total_kv, mode=MODES[mode], dtype=DTYPES[dtype],
                      causal=int(bool(causal)), qk_scale=float(qk_scale),
                      kv_len_normalize=int(kv_len_normalize), bias_kind=BIAS_KINDS[bias_kind],
                      num_buckets=int(num_buckets), split_slots=int(split_slots),
                      bwd_fuse=int(bwd_fuse), window=int(window))


def _workspace(problem: JfaProblem, backward: bool, device):
    import torch
    nbytes = jfa_workspace_bytes(problem, backward)
    if nbytes == 0:
        raise JfaError("jfa_workspace_bytes", _lib.JFA_ERR_INVALID_ARG)
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def _problem_of(q, k, q_offsets, mode, causal, bias_kind, num_buckets, qk_scale,
                kv_len_normalize, split_slots, dtype=None, bwd_fuse=-1,
                window=0) -> JfaProblem:
    import torch
    if dtype is None:
        dtype = {torch.float32: "f32", torch.bfloat16: "bf16", torch.uint8: "mxfp8"}[q.dtype]
    return make_problem(q_offsets.shape[0] - 1, q.shape[1], q.shape[2], q.shape[0], k.shape[0],
                        mode=mode, dtype=dtype, causal=causal, qk_scale=qk_scale,
                        kv_len_normalize=kv_len_normalize, bias_kind=bias_kind,
                        num_buckets=num_buckets, split_slots=split_slots, bwd_fuse=bwd_fuse,
                        window=window)


def forward(q, k, v, q_offsets, kv_offsets, *, mode: str = "softmax", causal: bool = False,
            bias=None, bias_kind: str = "none", num_buckets: int = 64, qk_scale: float = 0.0,
            kv_len_normalize: int = -1, split_slots: int = 0, q_scale=None, k_scale=None,
            v_scale=None, workspace=None, out=None, window: int = 0):
    """Returns (o, lse); lse is None for GDPA.  MXFP8: q/k/v are uint8 codes plus scales.
    window > 0: sliding-window attention (see jfa_problem.window)."""
    import torch
    problem = _problem_of(q, k, q_offsets, mode, causal, bias_kind, num_buckets, qk_scale,
                          kv_len_normalize, split_slots, window=window)
    odtype = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
    o = out if out is not None else torch.empty(q.shape, dtype=odtype, device=q.device)
    lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device) \
        if mode == "softmax" else None
    if workspace is None:
        workspace, nbytes = _workspace(problem, False, q.device)
    else:
        nbytes = workspace.numel()
    jfa_forward(problem, q, k, v, q_scale, k_scale, v_scale, q_offsets, kv_offsets, bias, o, lse,
                workspace, nbytes)
    return o, lse


def backward(q, k, v, o, lse, dout, q_offsets, kv_offsets, *, mode: str = "softmax",
             causal: bool = False, bias=None, bias_kind: str = "none", num_buckets: int = 64,
             qk_scale: float = 0.0, kv_len_normalize: int = -1, workspace=None, bwd_fuse=-1,
             window: int = 0):
    """Returns (dq, dk, dv), the gradients of <O, dout>."""
    import torch
    problem = _problem_of(q, k, q_offsets, mode, causal, bias_kind, num_buckets, qk_scale,
                          kv_len_normalize, 0, bwd_fuse=bwd_fuse, window=window)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    if workspace is None:
        workspace, nbytes = _workspace(problem, True, q.device)
    else:
        nbytes = workspace.numel()
    jfa_backward(problem, q, k, v, o, lse, dout, q_offsets, kv_offsets, bias, dq, dk, dv,
                 workspace, nbytes)
    return dq, dk, dv


def backward_mxfp8(q, k, v, q_scale, k_scale, v_scale, o, lse, dout, dout_scale, q_offsets,
                   kv_offsets, *, mode: str = "softmax", causal: bool = False, bias=None,
                   bias_kind: str = "none", num_buckets: int = 64, qk_scale: float = 0.0,
                   kv_len_normalize: int = -1, workspace=None, bwd_fuse=-1, window: int = 0):
    """MXFP8 backward: q, k, v, dout are E4M3 codes with their E8M0 scales (jfa_quantize_mxfp8);
    o, lse from the MXFP8 forward.  Returns bf16 (dq, dk, dv)."""
    import torch
    problem = _problem_of(q, k, q_offsets, mode, causal, bias_kind, num_buckets, qk_scale,
                          kv_len_normalize, 0, dtype="mxfp8", bwd_fuse=bwd_fuse, window=window)
    dq = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.bfloat16, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.bfloat16, device=q.device)
    if workspace is None:
        workspace, nbytes = _workspace(problem, True, q.device)
    else:
        nbytes = workspace.numel()
    jfa_backward_mxfp8(problem, q, k, v, q_scale, k_scale, v_scale, o, lse, dout, dout_scale,
                       q_offsets, kv_offsets, bias, dq, dk, dv, workspace, nbytes)
    return dq, dk, dv


def backward_dbias(q, k, v, o, lse, dout, q_offsets, kv_offsets, bias, *, mode: str = "softmax",
                   causal: bool = False, bias_kind: str = "relpos", num_buckets: int = 64,
                   qk_scale: float = 0.0, kv_len_normalize: int = -1, workspace=None,
                   window: int = 0):
    """Returns (dq, dk, dv, dbias): dbias is fp32 [H, num_buckets] for a relative-position
    table and bf16 in the bias's layout for a dense bias (bf16 inputs only)."""
    import torch
    problem = _problem_of(q, k, q_offsets, mode, causal, bias_kind, num_buckets, qk_scale,
                          kv_len_normalize, 0, window=window)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dbias = torch.empty_like(bias)
    if workspace is None:
        workspace, nbytes = _workspace(problem, 2, q.device)
    else:
        nbytes = workspace.numel()
    jfa_backward_dbias(problem, q, k, v, o, lse, dout, q_offsets, kv_offsets, bias, dq, dk, dv,
                       dbias, workspace, nbytes)
    return dq, dk, dv, dbias


def lengths_to_offsets(lengths):
    """int32 lengths [B] on the GPU -> (offsets int32 [B+1], status int32 [1])."""
    import torch
    off = torch.empty(lengths.shape[0] + 1, dtype=torch.int32, device=lengths.device)
    status = torch.empty(1, dtype=torch.int32, device=lengths.device)
    jfa_lengths_to_offsets(lengths, lengths.shape[0], off, status=status)
    return off, status


def bias_offsets(q_lengths, kv_lengths=None):
    """int32 lengths [B] (and kv lengths [B], default: the same) on the GPU -> (offsets int32
    [B+1], dense-bias block offsets int64 [B+1], status int32 [1])."""
    import torch
    dev = q_lengths.device
    off = torch.empty(q_lengths.shape[0] + 1, dtype=torch.int32, device=dev)
    boff = torch.empty(q_lengths.shape[0] + 1, dtype=torch.int64, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    jfa_lengths_to_offsets(q_lengths, q_lengths.shape[0], off, boff, kv_lengths, status)
    return off, boff, status


def block_offsets(offsets, block: int, total_rows: int):
    """BlockAttention: device offsets int32 [B+1] -> (refined offsets int32 [B'+1], B',
    status int32 [1]) with B' = B + total_rows // block (trailing samples empty).  Run the
    attention calls with batch B' and the refined offsets on both sides."""
    import torch
    B = offsets.shape[0] - 1
    out_batch = B + int(total_rows) // int(block)
    out = torch.empty(out_batch + 1, dtype=torch.int32, device=offsets.device)
    status = torch.empty(1, dtype=torch.int32, device=offsets.device)
    jfa_block_offsets(offsets, B, block, out, out_batch, status)
    return out, out_batch, status


def quantize_mxfp8(x):
    """bf16 [..., d] -> (E4M3 codes uint8 [..., d], E8M0 scales uint8 [..., d/32])."""
    import torch
    d = x.shape[-1]
    rows = x.numel() // d
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty(tuple(x.shape[:-1]) + (d // 32,), dtype=torch.uint8, device=x.device)
    jfa_quantize_mxfp8(x, rows, d, codes, scales)
    return codes, scales


def rmsnorm_quantize_mxfp8(x, weight=None, n: Optional[int] = None, eps: float = 1e-6):
    """bf16 [..., d] -> RMS-normalised over groups of n consecutive elements (default: the last
    dimension), times weight (fp32 [n] or None), then MXFP8: (codes uint8 [..., d], scales
    uint8 [..., d/32])."""
    import torch
    n = x.shape[-1] if n is None else n
    groups = x.numel() // n
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty(tuple(x.shape[:-1]) + (x.shape[-1] // 32,), dtype=torch.uint8,
                         device=x.device)
    jfa_rmsnorm_quantize_mxfp8(x, weight, groups, n, eps, codes, scales)
    return codes, scales


def build_schedule(problem: JfaProblem, q_offsets, kv_offsets, capacity: Optional[int] = None):
    """Runs only the tile scheduler; returns the lists as CPU int tensors."""
    import torch
    dev = q_offsets.device
    cap = capacity or int(problem.total_q + problem.total_kv + 4 * problem.batch + 4096)
    fwd = torch.zeros((cap, 4), dtype=torch.int32, device=dev)
    fslot = torch.zeros(cap, dtype=torch.int32, device=dev)
    comb = torch.zeros((cap, 4), dtype=torch.int32, device=dev)
    bq = torch.zeros((cap, 4), dtype=torch.int32, device=dev)
    bk = torch.zeros((cap, 4), dtype=torch.int32, device=dev)
    counts = torch.zeros(8, dtype=torch.int32, device=dev)
    ws, nbytes = _workspace(problem, False, dev)
    jfa_build_schedule(problem, q_offsets, kv_offsets, fwd, fslot, comb, bq, bk, counts, cap, ws,
                       nbytes)
    c = counts.cpu().tolist()
    return dict(fwd=fwd[:c[0]].cpu(), fwd_slot=fslot[:c[0]].cpu(), combine=comb[:c[1]].cpu(),
                bwd_q=bq[:c[2]].cpu(), bwd_kv=bk[:c[3]].cpu(), split_threshold=c[4],
                slots_used=c[5], status=c[6])


def _autograd():
    import torch

    class JaggedAttention(torch.autograd.Function):
        """Autograd wrapper: forward and backward both run libjfa kernels."""

        @staticmethod
        def forward(ctx, q, k, v, q_offsets, kv_offsets, bias, opts):
            o, lse = forward(q, k, v, q_offsets, kv_offsets, bias=bias, **opts)
            ctx.save_for_backward(q, k, v, o, lse if lse is not None else o, q_offsets,
                                  kv_offsets)
            ctx.bias = bias
            ctx.opts = opts
            ctx.has_lse = lse is not None
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse, qo, ko = ctx.saved_tensors
            opts = {key: val for key, val in ctx.opts.items() if key != "split_slots"}
            lse = lse if ctx.has_lse else None
            if ctx.bias is not None and ctx.needs_input_grad[5]:
                # a trained bias: its gradient comes from the backward with dbias (bf16 only)
                if q.dtype != torch.bfloat16:
                    raise NotImplementedError(
                        "the bias gradient is built for bf16 inputs; got " + str(q.dtype))
                dopts = {key: val for key, val in opts.items() if key != "bwd_fuse"}
                dq, dk, dv, dbias = backward_dbias(q, k, v, o, lse, do.contiguous(), qo, ko,
                                                   ctx.bias, **dopts)
                return dq, dk, dv, None, None, dbias, None
            dq, dk, dv = backward(q, k, v, o, lse, do.contiguous(), qo, ko, bias=ctx.bias,
                                  **opts)
            return dq, dk, dv, None, None, None, None

    return JaggedAttention


class _Lazy:
    _cls = None

    def __getattr__(self, name):
        if _Lazy._cls is None:
            _Lazy._cls = _autograd()
        return getattr(_Lazy._cls, name)


JaggedAttention = _Lazy()
