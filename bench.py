"""Benchmark: jagged attention forward + backward on one MI355X.

One step = the whole hot path over one synthetic batch: offsets from lengths, tile lists,
forward (with split-KV combine), softmax preprocess, dK/dV and dQ passes.  The headline
workload is causal jagged self-attention over user histories with a relative-position bias
(B=64, lengths log-normal median 512 clipped to [16, 4096], H=4, d=128, bf16, seed 2).
Inputs are resident in HBM before the timed region.  Every step is timed with HIP events on
the stream, after a 512 MB write that flushes the 256 MB MALL; the median over the steps is the
reported time (p10 and p90 beside it, and back-to-back steps as a secondary).  The same step
captured once as a HIP graph (checked bit-exact against an eager step) is timed too, and so are
the forward and the backward on their own.  Defaults: 10 warm-up steps, 50 timed.  Prints ONE
JSON line.

Useful FLOPs count only visible (query, key) pairs: 4*d per pair forward, 10*d backward.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "jagged attention fwd+bwd useful TFLOP/s and % of MI355X MFMA peak"
PEAK_BF16_TFLOPS = 2516.6        # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5033.2         # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
BLOCK_ROWS = 256                 # BlockAttention block size / sliding window of the extra lines


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_pairs(q_lens, kv_lens, causal, window=0):
    """Visible (query, key) pairs per sample: key j is visible to query i iff j <= i + (m - n)
    (causal) and |i + (m - n) - j| < window (window > 0)."""
    n = q_lens.astype(np.int64)
    m = kv_lens.astype(np.int64)
    if not causal and not window:
        return n * m
    out = np.zeros_like(n)
    for b in range(len(n)):
        a = np.arange(n[b]) + m[b] - n[b]          # aligned position of every query
        lo = np.zeros_like(a) if not window else a - window + 1
        hi = np.full_like(a, m[b]) if not window else a + window
        if causal:
            hi = np.minimum(hi, a + 1)
        out[b] = np.clip(np.minimum(hi, m[b]) - np.maximum(lo, 0), 0, None).sum()
    return out


class Workload:
    """Device buffers and preallocated outputs for one jfa_synth case."""

    def __init__(self, case, with_backward=True, block=0, dbias=False, window=0):
        import torch
        import jagged_attention_amd as jfa
        self.case = case
        self.block = block
        self.window = window
        # dbias: the backward also returns the bias gradient (jfa_backward_dbias)
        self.want_dbias = bool(dbias) and case.bias is not None and with_backward
        dev = torch.device("cuda:0")
        self.q = case.q.to(dev)
        self.k = case.k.to(dev)
        self.v = case.v.to(dev)
        self.bias = None if case.bias is None else case.bias.to(dev)
        self.dout = case.dout.to(dev) if (with_backward and case.dout is not None) else None
        self.q_lens = torch.as_tensor(case.q_lens, dtype=torch.int32, device=dev)
        self.kv_lens = torch.as_tensor(case.kv_lens, dtype=torch.int32, device=dev)
        # self-attention: one length array, so one offsets array serves queries and keys
        self.self_attn = bool(np.array_equal(case.q_lens, case.kv_lens))
        self.qo = torch.empty(case.batch + 1, dtype=torch.int32, device=dev)
        self.ko = torch.empty(case.batch + 1, dtype=torch.int32, device=dev)
        self.status = torch.zeros(2, dtype=torch.int32, device=dev)
        self.fp8 = case.dtype == "mxfp8"
        if self.fp8:
            # the quantiser is part of the MXFP8 input path and runs inside every step
            self.qc, self.qs = jfa.quantize_mxfp8(self.q)
            self.kc, self.ks = jfa.quantize_mxfp8(self.k)
            self.vc, self.vs = jfa.quantize_mxfp8(self.v)
            if self.dout is not None:
                self.doc, self.dos = jfa.quantize_mxfp8(self.dout)
        batch = case.batch
        if block:
            # BlockAttention: the attention calls run on the refined batch of blocks
            batch = case.batch + case.total_q // block
            self.boff = torch.empty(batch + 1, dtype=torch.int32, device=dev)
        self.batch = batch
        self.problem = jfa.make_problem(batch, case.heads, case.head_dim, case.total_q,
                                        case.total_kv, mode=case.mode,
                                        dtype=case.dtype, causal=case.causal,
                                        bias_kind=case.bias_kind, num_buckets=case.num_buckets,
                                        window=window)
        odt = torch.float32 if case.dtype == "f32" else torch.bfloat16
        self.o = torch.empty(self.q.shape, dtype=odt, device=dev)
        self.lse = torch.empty((case.heads, case.total_q), dtype=torch.float32, device=dev) \
            if case.mode == "softmax" else None
        nf = jfa.jfa_workspace_bytes(self.problem, False)
        self.ws_f = torch.empty(nf, dtype=torch.uint8, device=dev)
        self.nf = nf
        self.with_backward = self.dout is not None
        if self.with_backward:
            nb = jfa.jfa_workspace_bytes(self.problem, 2 if self.want_dbias else 1)
            self.ws_b = torch.empty(nb, dtype=torch.uint8, device=dev)
            self.nb = nb
            self.dq = torch.empty_like(self.q)       # bf16 also for MXFP8 inputs
            self.dk = torch.empty_like(self.k)
            self.dv = torch.empty_like(self.v)
            self.dbias = torch.empty_like(self.bias) if self.want_dbias else None
        if block:
            bl = np.array([min(block, n - s) for n in case.q_lens for s in range(0, n, block)],
                          dtype=np.int64)
            pairs = visible_pairs(bl, bl, case.causal) * case.heads
        else:
            pairs = visible_pairs(case.q_lens, case.kv_lens, case.causal, window) * case.heads
        self.pairs = int(pairs.sum())
        d = case.head_dim
        self.fwd_flops = 4.0 * d * self.pairs
        self.bwd_flops = 10.0 * d * self.pairs if self.with_backward else 0.0

    def step(self):
        self.step_forward()
        if self.with_backward:
            self.step_backward()

    def step_forward(self):
        """Offsets (and the BlockAttention refinement), the MXFP8 quantiser (with dO when the
        step has a backward: one launch for all), and the forward."""
        import jagged_attention_amd as jfa
        jfa.jfa_lengths_to_offsets(self.q_lens, self.case.batch, self.qo, status=self.status[0:1])
        if self.block:
            # self-attention split into blocks: one offsets array, refined, on both sides
            jfa.jfa_block_offsets(self.qo, self.case.batch, self.block, self.boff, self.batch,
                                  self.status[1:2])
            jfa.jfa_forward(self.problem, self.q, self.k, self.v, None, None, None, self.boff,
                            self.boff, self.bias, self.o, self.lse, self.ws_f, self.nf)
            return
        ko = self.qo
        if not self.self_attn:
            jfa.jfa_lengths_to_offsets(self.kv_lens, self.case.batch, self.ko,
                                       status=self.status[1:2])
            ko = self.ko
        if self.fp8:
            d = self.case.head_dim
            todo = [(self.q, self.qc, self.qs), (self.k, self.kc, self.ks),
                    (self.v, self.vc, self.vs)]
            if self.with_backward:
                todo.append((self.dout, self.doc, self.dos))
            # one launch for all of them
            jfa.jfa_quantize_mxfp8_batch([t[0] for t in todo], [t[0].numel() // d for t in todo],
                                         d, [t[1] for t in todo], [t[2] for t in todo])
            jfa.jfa_forward(self.problem, self.qc, self.kc, self.vc, self.qs, self.ks, self.vs,
                            self.qo, ko, self.bias, self.o, self.lse, self.ws_f, self.nf)
            return
        jfa.jfa_forward(self.problem, self.q, self.k, self.v, None, None, None, self.qo, ko,
                        self.bias, self.o, self.lse, self.ws_f, self.nf)

    def step_backward(self):
        """The backward (scheduler with D, both passes; the bias gradient when asked), on the
        offsets and forward outputs of the last step_forward."""
        import jagged_attention_amd as jfa
        if self.block:
            jfa.jfa_backward(self.problem, self.q, self.k, self.v, self.o, self.lse, self.dout,
                             self.boff, self.boff, self.bias, self.dq, self.dk, self.dv,
                             self.ws_b, self.nb)
            return
        ko = self.qo if self.self_attn else self.ko
        if self.fp8:
            jfa.jfa_backward_mxfp8(self.problem, self.qc, self.kc, self.vc, self.qs, self.ks,
                                   self.vs, self.o, self.lse, self.doc, self.dos, self.qo, ko,
                                   self.bias, self.dq, self.dk, self.dv, self.ws_b, self.nb)
        elif self.want_dbias:
            jfa.jfa_backward_dbias(self.problem, self.q, self.k, self.v, self.o, self.lse,
                                   self.dout, self.qo, ko, self.bias, self.dq, self.dk, self.dv,
                                   self.dbias, self.ws_b, self.nb)
        else:
            jfa.jfa_backward(self.problem, self.q, self.k, self.v, self.o, self.lse, self.dout,
                             self.qo, ko, self.bias, self.dq, self.dk, self.dv, self.ws_b,
                             self.nb)

    def algorithmic_bytes(self):
        """HBM bytes the method must move per step (inputs once, outputs once): forward reads
        Q, K, V (and the bias) and writes O (+ LSE for softmax); backward reads Q, K, V, dO
        (+ O and LSE for softmax, + the bias) and writes dQ, dK, dV."""
        c = self.case
        el = 1 if c.dtype == "mxfp8" else (4 if c.dtype == "f32" else 2)
        sc = (1.0 / 32) if c.dtype == "mxfp8" else 0.0
        qb = c.total_q * c.heads * c.head_dim * (el + sc)
        kb = c.total_kv * c.heads * c.head_dim * (el + sc)
        ob = c.total_q * c.heads * c.head_dim * (4 if c.dtype == "f32" else 2)
        lse = c.total_q * c.heads * 4 if c.mode == "softmax" else 0
        bias = 0 if self.bias is None else self.bias.numel() * self.bias.element_size()
        fwd = qb + 2 * kb + bias + ob + lse
        bwd = 0
        if self.with_backward:
            # dO in the input format (codes + scales for MXFP8), O and the gradients bf16/fp32
            ib = 2 if c.dtype == "mxfp8" else el
            reads = 2 * qb + 2 * kb + bias + ((ob + lse) if c.mode == "softmax" else 0)
            grads = (c.total_q + 2 * c.total_kv) * c.heads * c.head_dim * ib
            bwd = reads + grads
        return fwd, bwd

    def padded_flops(self):
        """FLOPs of the same batch padded to its longest sample (what a dense kernel would
        execute): every sample takes max q_len queries and max kv_len keys."""
        c = self.case
        n = int(np.max(c.q_lens)) if c.batch else 0
        m = int(np.max(c.kv_lens)) if c.batch else 0
        pairs = c.batch * c.heads * int(visible_pairs(np.array([n]), np.array([m]),
                                                      c.causal)[0])
        per = (4.0 + (10.0 if self.with_backward else 0.0)) * c.head_dim
        return per * pairs


def outputs(w):
    """The step's outputs (forward and backward), for comparing a graph replay with eager."""
    out = [w.o] + ([w.lse] if w.lse is not None else [])
    if w.with_backward:
        out += [w.dq, w.dk, w.dv]
    if w.want_dbias:
        out.append(w.dbias)
    return out


def capture_step(w):
    """Captures one step into a HIP graph (torch.cuda.CUDAGraph) after checking that its replay
    reproduces an eager step bit for bit (every kernel here is deterministic)."""
    import torch
    torch.cuda.synchronize()
    w.step()
    torch.cuda.synchronize()
    want = [t.clone() for t in outputs(w)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w.step()
    for t in outputs(w):
        t.zero_()
    g.replay()
    torch.cuda.synchronize()
    for a, b in zip(outputs(w), want):
        if not torch.equal(a, b):
            raise RuntimeError("graph replay differs from the eager step")
    return g


FLUSH_BYTES = 512 << 20           # twice the 256 MB MALL (Infinity Cache) of MI355X


class Flusher:
    """Writes a 512 MB scratch buffer on the current stream, so no input of the next step is
    left in the MALL or the L2s (a fill kernel: every line of it is written)."""

    def __init__(self):
        import torch
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda:0")
        self.k = 0

    def __call__(self):
        self.k += 1
        self.buf.fill_(self.k)


def _timed(fn, steps, warmup, flush=None):
    """Per-step device times (ms) of fn() from HIP events on the current stream; with flush, the
    MALL is flushed before every step, outside the events."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        if flush is not None:
            flush()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev])


def stats(ms):
    return dict(median=float(np.median(ms)), p10=float(np.percentile(ms, 10)),
                p90=float(np.percentile(ms, 90)), mean=float(np.mean(ms)))


def time_graph(g, steps, warmup, flush=None):
    return _timed(g.replay, steps, warmup, flush)


def time_steps(w, steps, warmup, flush=None):
    return _timed(w.step, steps, warmup, flush)


def kernel_times(w, steps, flush=None):
    """Average device time per launch of each library kernel (HIP events the library records
    on its own stream around every launch), over `steps` steps, each after a MALL flush."""
    import torch
    import jagged_attention_amd as jfa
    jfa.jfa_kernel_timing_reset()
    for _ in range(steps):
        if flush is not None:
            flush()
        jfa.jfa_set_kernel_timing(True)
        w.step()
        jfa.jfa_set_kernel_timing(False)
    torch.cuda.synchronize()
    names = ("jfa_offsets", "jfa_block_offsets", "jfa_schedule", "jfa_quant_mxfp8",
             "jfa_fwd_bf16", "jfa_fwd_mxfp8", "jfa_fwd_f32", "jfa_fwd_combine",
             "jfa_bwd_kvq", "jfa_bwd_dkdv", "jfa_bwd_dq",
             "jfa_bwd_kvq_mxfp8", "jfa_bwd_dkdv_mxfp8", "jfa_bwd_dq_mxfp8",
             "jfa_bwd_dkdv_f32", "jfa_bwd_dq_f32",
             "jfa_dbias_zero", "jfa_dbias_dq", "jfa_dbias_reduce")
    # the library matches names by prefix: take the longer names' launches out of each total
    raw = {name: jfa.jfa_kernel_timing(name) for name in names}
    out = {}
    for name in names:
        ms, n = raw[name]
        for other in names:
            if other != name and other.startswith(name):
                ms -= raw[other][0]
                n -= raw[other][1]
        if n:
            out[name] = dict(avg_ms=ms / n, launches=n)
    jfa.jfa_kernel_timing_reset()
    return out


# MFMA flops per visible pair (multiples of d) credited to each kernel.  Useful work: 4 d
# forward (QK^T, PV) and 10 d backward (S recompute, dP, dV, dQ, dK); the key-stationary pass
# does S, dP, dV, dK (8 d), the query-stationary pass adds only dQ (2 d) of useful work, so when
# both run in one launch it is credited 10 d.  Executed work counts the query-stationary pass's
# recompute of S and dP too (6 d; 14 d for the shared launch).
USEFUL_FLOPS_PER_PAIR = {"jfa_fwd_bf16": 4, "jfa_fwd_mxfp8": 4, "jfa_bwd_kvq": 10,
                         "jfa_bwd_dkdv": 8, "jfa_bwd_dq": 2, "jfa_dbias_dq": 2,
                         "jfa_bwd_kvq_mxfp8": 10, "jfa_bwd_dkdv_mxfp8": 8,
                         "jfa_bwd_dq_mxfp8": 2}
EXECUTED_FLOPS_PER_PAIR = {"jfa_fwd_bf16": 4, "jfa_fwd_mxfp8": 4, "jfa_bwd_kvq": 14,
                           "jfa_bwd_dkdv": 8, "jfa_bwd_dq": 6, "jfa_dbias_dq": 6,
                           "jfa_bwd_kvq_mxfp8": 14, "jfa_bwd_dkdv_mxfp8": 8,
                           "jfa_bwd_dq_mxfp8": 6}
# kernels whose products run on the fp8 MFMA (QK^T of the MXFP8 forward); every other product,
# the MXFP8 backward's included, runs on bf16 MFMA
FP8_MFMA_KERNELS = ("jfa_fwd_mxfp8",)


def traffic_for(kernel, workload):
    """HBM traffic of `kernel` per launch on `workload` from the committed counter summary, if
    current."""
    from jagged_attention_amd.traffic import file_tag
    path = os.path.join(ROOT, "profiles", f"traffic_{file_tag(workload)}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    from jagged_attention_amd.traffic import source_hash
    ent = rec.get("kernels", {}).get(kernel)
    if not ent or ent.get("source_hash") != source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_timing(case, target_s):
    """The oracle (fp64, all host threads) on a bounded sample of `case`: samples taken in batch
    order while the estimated time fits `target_s` (calibrated on the cheapest samples).
    Returns useful TFLOP/s of the fwd (+bwd) pass and the sample description."""
    import oracle
    oracle.build()
    back = case.dout is not None
    pairs = visible_pairs(case.q_lens, case.kv_lens, case.causal)
    per_pair = (4.0 + (10.0 if back else 0.0)) * case.head_dim * case.heads
    qo = np.concatenate([[0], np.cumsum(case.q_lens.astype(np.int64))])
    ko = np.concatenate([[0], np.cumsum(case.kv_lens.astype(np.int64))])
    H = case.heads
    bo = np.concatenate([[0], np.cumsum(case.q_lens.astype(np.int64) *
                                        case.kv_lens.astype(np.int64))]) * H

    def run(idx):
        idx = np.asarray(idx, dtype=np.int64)
        rq = np.concatenate([np.arange(qo[b], qo[b + 1]) for b in idx] + [np.zeros(0, np.int64)])
        rk = np.concatenate([np.arange(ko[b], ko[b + 1]) for b in idx] + [np.zeros(0, np.int64)])
        bias = case.bias
        if case.bias_kind == "dense":
            bias = np.concatenate([case.bias[int(bo[b]):int(bo[b + 1])].float().numpy()
                                   for b in idx] + [np.zeros(0, np.float32)])
        kw = dict(mode=case.mode, causal=case.causal, bias=bias, bias_kind=case.bias_kind,
                  num_buckets=case.num_buckets)
        q, k, v = case.q[rq], case.k[rk], case.v[rk]
        t0 = time.perf_counter()
        oracle.forward(q, k, v, case.q_lens[idx], case.kv_lens[idx], **kw)
        if back:
            oracle.backward(q, k, v, case.dout[rq], case.q_lens[idx], case.kv_lens[idx], **kw)
        return time.perf_counter() - t0

    order = np.arange(case.batch)
    cheap = order[np.argsort(pairs, kind="stable")][:min(8, case.batch)]
    t_cal = run(cheap)
    rate = per_pair * max(int(pairs[cheap].sum()), 1) / max(t_cal, 1e-6)   # flop/s
    budget = rate * target_s
    chosen, acc = [], 0.0
    for b in order:
        f = per_pair * pairs[b]
        if acc + f > budget and chosen:
            continue
        chosen.append(int(b))
        acc += f
    t = run(chosen)
    flops = per_pair * pairs[chosen].sum()
    return dict(value=float(flops / t / 1e12), unit="TFLOP/s", cores=oracle.max_threads(),
                kind="oracle", cpu_model=cpu_model(),
                sample=f"{len(chosen)} of {case.batch} samples of {case.name} in batch order "
                       f"({int(pairs[chosen].sum()) * H} visible (query, key, head) triples, "
                       f"{'fwd+bwd' if back else 'fwd'} in fp64, {t:.1f} s)")


def bench_config(cfg, steps, warmup, seed=None, block=0, dbias=False, flush=None, window=0,
                 with_dout=None):
    from jfa_synth import make_case
    case = make_case(cfg, seed, with_dout=with_dout)
    w = Workload(case, block=block, dbias=dbias, window=window)
    t_fl = stats(time_steps(w, steps, warmup, flush))          # MALL flushed before every step
    t_hot = stats(time_steps(w, steps, 1))                     # back to back (secondary)
    # the forward and the backward on their own (each flushed; the backward reuses the last
    # forward's outputs)
    t_fwd = stats(_timed(w.step_forward, steps, 1, flush))
    t_bwd = stats(_timed(w.step_backward, steps, 1, flush)) if w.with_backward else None
    # the same step replayed as one HIP graph (no per-launch host work): reported beside it
    w.graph = capture_step(w)
    t_graph = stats(time_graph(w.graph, steps, 1, flush))
    flops = w.fwd_flops + w.bwd_flops
    peak = PEAK_FP8_TFLOPS if case.dtype == "mxfp8" else PEAK_BF16_TFLOPS
    fb, bb = w.algorithmic_bytes()
    intensity = flops / (fb + bb)
    ceiling = min(peak, intensity * PEAK_HBM_GBS / 1000.0)
    sec = t_fl["median"] * 1e-3
    tf = flops / sec / 1e12
    padded = w.padded_flops()
    name = case.name if not block else f"block{block}-" + case.name
    if window:
        name = f"window{window}-" + name
    if case.dtype == "mxfp8" and w.with_backward:
        name += "+bwd"
    if w.want_dbias:
        name += "+dbias"
    return w, dict(workload=name, seed=case.seed, ms_per_step=t_fl["median"],
                   ms_p10=t_fl["p10"], ms_p90=t_fl["p90"],
                   unflushed_ms_per_step=t_hot["median"],
                   fwd_ms=t_fwd["median"], bwd_ms=None if t_bwd is None else t_bwd["median"],
                   fwd_tflops=w.fwd_flops / (t_fwd["median"] * 1e-3) / 1e12,
                   bwd_tflops=None if t_bwd is None else
                   w.bwd_flops / (t_bwd["median"] * 1e-3) / 1e12,
                   graph_ms_per_step=t_graph["median"], tflops=tf,
                   frac_of_mfma_peak=tf / peak, roofline_ceiling_tflops=ceiling,
                   frac_of_roofline=tf / ceiling, useful_gflop=flops / 1e9,
                   algorithmic_mb=(fb + bb) / 1e6,
                   padded_gflop=padded / 1e9,
                   padding_waste_frac=(1.0 - flops / padded) if padded > 0 else 0.0,
                   passes="fwd" if not w.with_backward else "fwd+bwd")


def kernel_work(w):
    """Per-launch work of each attention kernel of the step: {kernel: (useful flops, executed
    flops, algorithmic HBM bytes)}.  The backward's samples fall into three classes (the
    scheduler's test, from the tile configuration): one query tile (the query-stationary pass
    also writes dK, dV: 10 d useful per pair), else one key tile at d = 64 (the key-stationary
    pass also writes dQ: 10 d), else both passes (8 d + 2 d useful, 8 d + 6 d executed).  Bytes
    count every tensor a kernel must read or write once (per class: Q, dO, LSE and D, K, V, the
    dense bias; the gradients it writes)."""
    import jagged_attention_amd as jfa
    c = w.case
    d, H = c.head_dim, c.heads
    if w.block:
        ql = np.array([min(w.block, n - s) for n in c.q_lens for s in range(0, n, w.block)],
                      dtype=np.int64)
        kl = ql.copy()
    else:
        ql = c.q_lens.astype(np.int64)
        kl = c.kv_lens.astype(np.int64)
    pairs = visible_pairs(ql, kl, c.causal, w.window).astype(np.float64) * H
    tc = jfa.jfa_tile_config(w.problem)
    fuse = 0 if w.want_dbias else tc["fuse"]           # the bias-gradient call runs both passes
    one_q = bool(fuse & 1) & (ql > 0) & (ql <= tc["bq_bm"])
    one_k = ~one_q & bool(fuse & 2) & (kl > 0) & (kl <= tc["bk_bn"])
    two = ~one_q & ~one_k
    es = (1 + 1 / 32) if c.dtype == "mxfp8" else (4 if c.dtype == "f32" else 2)
    gs = 4 if c.dtype == "f32" else 2                  # output / gradient element size
    qb = ql * H * d * es
    kb = kl * H * d * es
    rows = ql * H * 8 if c.mode == "softmax" else 0    # LSE and D (fp32)
    bias = ql * kl * H * 2 if c.bias_kind == "dense" else 0
    dq, dkv = ql * H * d * gs, 2 * kl * H * d * gs
    if w.want_dbias:
        dq = dq + bias                                 # the dense bias gradient, written once
    reads = 2 * qb + 2 * kb + rows + bias              # Q, dO, LSE / D, K, V, bias
    q_cls = one_q | two
    k_cls = one_k | two
    work = {
        "fwd": (4 * d * pairs.sum(), 4 * d * pairs.sum(),
                (qb + 2 * kb + bias + ql * H * d * gs + (ql * H * 4 if c.mode == "softmax"
                                                         else 0)).sum()),
        "dq": ((10 * d * pairs[one_q]).sum() + (2 * d * pairs[two]).sum(),
               (10 * d * pairs[one_q]).sum() + (6 * d * pairs[two]).sum(),
               np.sum(np.where(q_cls, reads + dq, 0) + np.where(one_q, dkv, 0))),
        "dkdv": ((10 * d * pairs[one_k]).sum() + (8 * d * pairs[two]).sum(),
                 (10 * d * pairs[one_k]).sum() + (8 * d * pairs[two]).sum(),
                 np.sum(np.where(k_cls, reads + dkv, 0) + np.where(one_k, dq, 0))),
    }
    kvq = (work["dq"][0] + work["dkdv"][0], work["dq"][1] + work["dkdv"][1],
           work["dq"][2] + work["dkdv"][2])
    work["kvq"] = kvq
    out = {}
    for name in USEFUL_FLOPS_PER_PAIR:
        part = ("fwd" if "fwd" in name else "kvq" if "kvq" in name
                else "dkdv" if "dkdv" in name else "dq")
        out[name] = work[part]
    return out


def roofline_of(w, kt):
    """Roofline record of the dominant attention kernel of the step (largest total time):
    useful FLOP/s against the MFMA peak of its dtype, or algorithmic HBM GB/s against 8 TB/s
    when its useful flops per algorithmic byte are below the ridge point (peak / 8 TB/s)."""
    cand = {k: v for k, v in kt.items() if k in USEFUL_FLOPS_PER_PAIR}
    if not cand:
        return None
    dom = max(cand, key=lambda k: cand[k]["avg_ms"] * cand[k]["launches"])
    useful, executed, nbytes = kernel_work(w)[dom]
    nbytes = max(float(nbytes), 1.0)
    sec = cand[dom]["avg_ms"] * 1e-3
    peak = PEAK_FP8_TFLOPS if dom in FP8_MFMA_KERNELS else PEAK_BF16_TFLOPS
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    rec = dict(kernel=dom, traffic=traffic_for(dom, w.case.name),
               flops_per_launch=int(useful), executed_flops_per_launch=int(executed),
               bytes_per_launch=int(nbytes), flops_per_byte=round(useful / nbytes, 1),
               mfma_frac=round(useful / sec / 1e12 / peak, 4),
               executed_frac=round(executed / sec / 1e12 / peak, 4),
               hbm_frac=round(nbytes / sec / 1e9 / PEAK_HBM_GBS, 4),
               avg_ms=cand[dom]["avg_ms"])
    if useful / nbytes < ridge:
        gbs = nbytes / sec / 1e9
        rec.update(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                   frac=round(gbs / PEAK_HBM_GBS, 4))
    else:
        tf = useful / sec / 1e12
        rec.update(bound="mfma", achieved=round(tf, 2), peak=peak, unit="TFLOP/s",
                   frac=round(tf / peak, 4))
    return {k: rec[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")} | rec


def bench_norm_quant(cfg=5, reps=10):
    """The fused RMS normalisation + MXFP8 quantiser (one group per row and head, n = d) on the
    MXFP8 workload's Q, K and V, against the plain quantiser on the same tensors (HIP events)."""
    import torch
    import jagged_attention_amd as jfa
    from jfa_synth import make_case
    case = make_case(cfg)
    d = case.head_dim
    xs = [t.to("cuda:0") for t in (case.q, case.k, case.v)]
    outs = [(torch.empty(x.shape, dtype=torch.uint8, device=x.device),
             torch.empty(tuple(x.shape[:-1]) + (d // 32,), dtype=torch.uint8, device=x.device))
            for x in xs]
    w = torch.ones(d, dtype=torch.float32, device="cuda:0")
    elems = sum(x.numel() for x in xs)

    def run(fused):
        for x, (c, sc) in zip(xs, outs):
            if fused:
                jfa.jfa_rmsnorm_quantize_mxfp8(x, w, x.numel() // d, d, 1e-6, c, sc)
            else:
                jfa.jfa_quantize_mxfp8(x, x.numel() // d, d, c, sc)

    res = {}
    for name, fused in (("jfa_norm_quant_mxfp8", True), ("jfa_quant_mxfp8", False)):
        run(fused)
        torch.cuda.synchronize()
        jfa.jfa_kernel_timing_reset()
        jfa.jfa_set_kernel_timing(True)
        for _ in range(reps):
            run(fused)
        torch.cuda.synchronize()
        jfa.jfa_set_kernel_timing(False)
        ms, n = jfa.jfa_kernel_timing(name)
        jfa.jfa_kernel_timing_reset()
        sec = ms / reps * 1e-3                        # Q, K and V, one launch each
        gbs = elems * (2 + 1 + 1 / 32) / sec / 1e9    # bf16 read, codes + scales written
        res[name] = dict(us_for_qkv=round(sec * 1e6, 1), launches=n, gbs=round(gbs, 1),
                         frac_of_hbm=round(gbs / PEAK_HBM_GBS, 4))
    del xs, outs
    torch.cuda.empty_cache()
    return dict(workload=case.name + "-qkv-norm-quant", elements=elems, group=d,
                algorithmic_bytes_per_element=2 + 1 + 1 / 32, **res)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baselines")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--config", type=int, default=2, help="headline workload (1..5)")
    ap.add_argument("--dbias", action="store_true",
                    help="the main workload's backward also returns the bias gradient")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the jagged attention path has no cross-GPU exchange).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import jagged_attention_amd as jfa
    jfa.load()

    if args.copy_mib > 0:
        # a plain copy of known size: what FETCH_SIZE / WRITE_SIZE read for it calibrates them
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] calibration copy: {args.copy_mib} MiB x 3")
    flush = Flusher()
    log(f"[bench] headline workload {args.config}: warmup {args.warmup}, steps {args.steps}")
    w, head = bench_config(args.config, args.steps, args.warmup, dbias=args.dbias, flush=flush)
    log(f"[bench] {head['workload']}: {head['ms_per_step']:.3f} ms/step (p10 "
        f"{head['ms_p10']:.3f}, p90 {head['ms_p90']:.3f}), {head['tflops']:.1f} TFLOP/s")
    kt = kernel_times(w, max(3, args.steps // 2), flush)
    log(f"[bench] kernel times: {json.dumps(kt)}")
    roof = roofline_of(w, kt)

    extra = {}
    if not args.no_extra:
        for cfg in (3, 4, 5):
            if cfg == args.config:
                continue
            log(f"[bench] workload {cfg}")
            wx, r = bench_config(cfg, max(3, args.steps // 2), 2, flush=flush)
            r["kernels"] = kernel_times(wx, 3, flush)
            r["roofline"] = roofline_of(wx, r["kernels"])
            if cfg == 5:
                # low-precision gate: the MXFP8 step (its three quantiser launches included)
                # against the bf16 forward on the same batch
                import copy
                cb = copy.copy(wx.case)
                cb.dtype = "bf16"
                del wx
                torch.cuda.empty_cache()
                wb = Workload(cb, with_backward=False)
                tb = stats(time_steps(wb, max(3, args.steps // 2), 2, flush))
                r["bf16_forward_ms"] = tb["median"]
                r["mxfp8_step_speedup_vs_bf16"] = tb["median"] / r["ms_per_step"]
                r["bf16_kernels"] = kernel_times(wb, 3, flush)
                wx = wb
            extra[f"workload_{cfg}"] = r
            del wx
            torch.cuda.empty_cache()
        # BlockAttention: the headline batch with every sample split into blocks of 256 rows
        log("[bench] block attention")
        wx, r = bench_config(2, max(3, args.steps // 2), 2, block=BLOCK_ROWS, flush=flush)
        r["kernels"] = kernel_times(wx, 3, flush)
        r["block_rows"] = BLOCK_ROWS
        extra["block_attention"] = r
        del wx
        torch.cuda.empty_cache()
        # MXFP8 training step: the MXFP8 workload with dO, quantiser (Q, K, V, dO), forward and
        # the MXFP8 backward
        log("[bench] mxfp8 fwd+bwd")
        wx, r = bench_config(5, max(3, args.steps // 2), 2, flush=flush, with_dout=True)
        r["kernels"] = kernel_times(wx, 3, flush)
        r["roofline"] = roofline_of(wx, r["kernels"])
        r["frac_of_bf16_mfma_peak"] = r["tflops"] / PEAK_BF16_TFLOPS
        extra["mxfp8_fwd_bwd"] = r
        del wx
        torch.cuda.empty_cache()
        # sliding window: the headline batch, every query seeing its last 256 keys
        log("[bench] sliding window")
        wx, r = bench_config(2, max(3, args.steps // 2), 2, window=BLOCK_ROWS, flush=flush)
        r["kernels"] = kernel_times(wx, 3, flush)
        r["roofline"] = roofline_of(wx, r["kernels"])
        r["window"] = BLOCK_ROWS
        extra["sliding_window"] = r
        del wx
        torch.cuda.empty_cache()
        # fused normalisation + MXFP8 quantisation of the MXFP8 workload's inputs
        log("[bench] fused norm + quant")
        extra["norm_quant"] = bench_norm_quant()
        # the headline step with the bias gradient (the relative-position table is trained)
        log("[bench] bias gradient")
        wx, r = bench_config(2, max(3, args.steps // 2), 2, dbias=True, flush=flush)
        r["kernels"] = kernel_times(wx, 3, flush)
        extra["bias_gradient"] = r
        del wx
        # the short-KV GELU workload with its dense bias trained (both passes: the bias gradient
        # is formed in the query-stationary pass)
        log("[bench] dense bias gradient")
        wx, r = bench_config(4, max(3, args.steps // 2), 2, dbias=True, flush=flush)
        r["kernels"] = kernel_times(wx, 3, flush)
        extra["bias_gradient_dense"] = r
        del wx
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        log("[bench] oracle CPU baseline")
        cpu = oracle_timing(w.case, 15.0)
        if not args.no_extra:
            from jfa_synth import make_case
            for cfg in (1, 2, 3, 4, 5):
                if cfg == args.config:
                    continue                  # the headline's oracle is cpu_baseline
                c = make_case(cfg)
                o = oracle_timing(c, 4.0)
                tgt = extra.setdefault(f"workload_{cfg}", {})
                tgt["oracle"] = o
                if "tflops" in tgt:
                    tgt["gpu_over_oracle"] = tgt["tflops"] / o["value"]

    case = w.case
    line = {
        "metric": METRIC,
        "value": round(head["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "ms_p10": round(head["ms_p10"], 4),
        "ms_p90": round(head["ms_p90"], 4),
        "unflushed_ms_per_step": round(head["unflushed_ms_per_step"], 4),
        "graph_ms_per_step": round(head["graph_ms_per_step"], 4),
        "fwd_ms": round(head["fwd_ms"], 4),
        "bwd_ms": None if head["bwd_ms"] is None else round(head["bwd_ms"], 4),
        "fwd_tflops": round(head["fwd_tflops"], 3),
        "bwd_tflops": None if head["bwd_tflops"] is None else round(head["bwd_tflops"], 3),
        "timing": "median of per-step HIP events, a 512 MB write flushing the MALL before each "
                  "step; unflushed_ms_per_step: back-to-back steps; graph_ms_per_step: the step "
                  "replayed as one HIP graph (checked bit-exact against an eager step); fwd_ms "
                  "and bwd_ms: the forward (with the offsets) and the backward (scheduler "
                  "included) timed on their own, each flushed",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if case.dtype == "bf16" else case.dtype,
        "data": "synthetic",
        "config": {"workload": head["workload"], "batch": case.batch, "heads": case.heads,
                   "head_dim": case.head_dim, "total_tokens": case.total_q,
                   "lengths": "log-normal median 512 clipped to [16, 4096]" if args.config == 2
                   else "see jfa_synth", "mode": case.mode, "causal": case.causal,
                   "bias": case.bias_kind, "seed": case.seed, "parallelism": "single GPU"},
        "mfma_peak_frac": round(head["frac_of_mfma_peak"], 4),
        "useful_gflop": round(head["useful_gflop"], 3),
        "padded_gflop": round(head["padded_gflop"], 3),
        "padding_waste_frac": round(head["padding_waste_frac"], 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kt,
        "other_workloads": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
