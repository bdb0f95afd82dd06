"""GPU parity of the MXFP8 backward (jfa_backward_mxfp8) against the oracle's backward on the
dequantised inputs.

MXFP8 attention is part of training ("Meta Enhances GEM Training Efficiency with Advanced
LLM-Scale Innovations", section "Leveraging Compute Efficiency through Customized Kernels"), with
selective higher precision where gradients are sensitive ("Meta GEM Training Efficiency: ...",
section "Bottleneck move 2").  Q, K, V and dO are quantised by the library's quantiser (bit-exact
with the oracle's), the forward and backward run on the codes, and the gradients are compared with
the fp64 oracle at the dequantised values.  The contract bound for MXFP8 results is relative-L2
5e-2; since the kernels dequantise exactly and keep P and dS in bf16, the bf16 bounds (max-abs
2e-2 beyond output and operand rounding, relative-L2 1e-2) are asserted as well."""
import numpy as np
import pytest
import torch

import oracle
from jfa_synth import custom_case, make_case
from tests.gpu_helpers import compare, device_case, say
from tests.helpers import rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import jagged_attention_amd as jfa
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    jfa.load()
    oracle.build()
    return jfa


def _dequant(c, s):
    return oracle.mxfp8_dequantize(c.cpu().numpy(), s.cpu().numpy())


def _check(name, got, want, cond, bf16_bounds=True):
    g = got.float().cpu().numpy()
    rl = rel_l2(g, want)
    say(f"  {name}: rel-L2 {rl:.3e} (MXFP8 bound 5e-2)")
    assert np.all(np.isfinite(g)) and rl <= 5e-2, f"{name}: rel-L2 {rl:.3g} above the MXFP8 bound"
    if bf16_bounds:
        compare(name, got, want, "bf16", cond=cond)


def _run_case(case, window=0, bf16_bounds=True):
    import jagged_attention_amd as jfa
    dc = device_case(case)
    qc, qs = jfa.quantize_mxfp8(dc["q"])
    kc, ks = jfa.quantize_mxfp8(dc["k"])
    vc, vs = jfa.quantize_mxfp8(dc["v"])
    doc, dos = jfa.quantize_mxfp8(dc["dout"])
    kw = dict(mode=case.mode, causal=case.causal, bias=dc["bias"], bias_kind=case.bias_kind,
              num_buckets=case.num_buckets, window=window)
    o, lse = jfa.forward(qc, kc, vc, dc["qo"], dc["ko"], q_scale=qs, k_scale=ks, v_scale=vs,
                         **kw)
    dq, dk, dv = jfa.backward_mxfp8(qc, kc, vc, qs, ks, vs, o, lse, doc, dos, dc["qo"],
                                    dc["ko"], **kw)
    torch.cuda.synchronize()
    assert dq.dtype == torch.bfloat16
    deq = [_dequant(c, s) for c, s in ((qc, qs), (kc, ks), (vc, vs), (doc, dos))]
    okw = dict(mode=case.mode, causal=case.causal, bias=case.bias, bias_kind=case.bias_kind,
               num_buckets=case.num_buckets, window=window)
    dq_ref, dk_ref, dv_ref = oracle.backward(deq[0], deq[1], deq[2], deq[3], case.q_lens,
                                             case.kv_lens, **okw)
    c = oracle.abs_terms(deq[0], deq[1], deq[2], deq[3], case.q_lens, case.kv_lens, **okw)
    _check("dQ", dq, dq_ref, c["dQ"], bf16_bounds)
    _check("dK", dk, dk_ref, c["dK"], bf16_bounds)
    _check("dV", dv, dv_ref, c["dV"], bf16_bounds)
    return dq, dk, dv


@pytest.mark.parametrize("mode,causal,bias_kind", [("softmax", True, "relpos"),
                                                    ("softmax", False, "none"),
                                                    ("silu", False, "dense"),
                                                    ("gelu", True, "none")])
@pytest.mark.parametrize("d", [128, 64])
def test_mxfp8_backward_parity(mode, causal, bias_kind, d):
    ql = [300, 17, 129, 0, 64, 520]
    kl = ql if causal else [200, 40, 9, 30, 64, 700]
    case = custom_case(ql, kl, 2, d, dtype="mxfp8", mode=mode, causal=causal,
                       bias_kind=bias_kind, seed=200 + d)
    say(f"[mxfp8 bwd] mode={mode} causal={causal} bias={bias_kind} d={d}")
    _run_case(case)


def test_mxfp8_backward_window_and_single_pass_classes():
    """A sliding window, and samples that take the single-pass classes (one query tile at
    64-row query tiles; one key tile at d = 64)."""
    case = custom_case([700, 5, 300], [700, 5, 300], 2, 128, dtype="mxfp8", mode="softmax",
                       causal=True, bias_kind="relpos", seed=210)
    say("[mxfp8 bwd] window 100")
    _run_case(case, window=100)
    short_q = custom_case([40, 64, 17, 55], [300, 90, 700, 45], 2, 128, dtype="mxfp8",
                          mode="silu", seed=211)
    say("[mxfp8 bwd] one query tile")
    _run_case(short_q)
    short_k = custom_case([256, 100, 256], [40, 64, 9], 2, 64, dtype="mxfp8", mode="gelu",
                          seed=212)
    say("[mxfp8 bwd] one key tile")
    _run_case(short_k)


def test_mxfp8_backward_block_scales_differ():
    """Each 32-element block along d at its own power-of-two magnitude: a scale applied to the
    wrong block or row of any of the four inputs shows up.  The MXFP8 bound (relative-L2) is the
    check here: with inputs magnified up to 16 times, softmax's D = dO.O is formed from the
    stored bf16 O, and its rounding (half an ulp of |O| up to ~60, times |dO|) moves dQ and dK
    by far more than 2e-2 in absolute terms while staying small relative to them."""
    ql = [200, 1, 77, 130]
    case = custom_case(ql, ql, 2, 128, dtype="mxfp8", causal=True, seed=213)
    rng = np.random.default_rng(214)
    for name in ("q", "k", "v", "dout"):
        x = getattr(case, name)
        e = rng.integers(-4, 5, size=(x.shape[0], x.shape[1], x.shape[2] // 32))
        f = torch.from_numpy(np.exp2(e).astype(np.float32)).repeat_interleave(32, dim=2)
        setattr(case, name, (x.float() * f).to(torch.bfloat16))
    say("[mxfp8 bwd] per-block scales")
    _run_case(case, bf16_bounds=False)


def test_mxfp8_backward_deterministic():
    import jagged_attention_amd as jfa
    case = custom_case([400, 77, 129], [400, 77, 129], 2, 128, dtype="mxfp8", causal=True,
                       bias_kind="relpos", seed=215)
    dc = device_case(case)
    q8 = [jfa.quantize_mxfp8(dc[x]) for x in ("q", "k", "v", "dout")]
    kw = dict(causal=True, bias=dc["bias"], bias_kind="relpos")
    o, lse = jfa.forward(q8[0][0], q8[1][0], q8[2][0], dc["qo"], dc["ko"], q_scale=q8[0][1],
                         k_scale=q8[1][1], v_scale=q8[2][1], **kw)
    args = (q8[0][0], q8[1][0], q8[2][0], q8[0][1], q8[1][1], q8[2][1], o, lse, q8[3][0],
            q8[3][1], dc["qo"], dc["ko"])
    a = jfa.backward_mxfp8(*args, **kw)
    b = jfa.backward_mxfp8(*args, **kw)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_mxfp8_backward_fullsize_sampled():
    """The MXFP8 workload (B=256, lengths to 8192) with dO, run by the benchmark's step
    (quantiser, forward, backward); the oracle on a sub-batch of chosen samples."""
    import bench
    from tests.test_gpu_fullsize import chosen_samples, rows
    case = make_case(5, with_dout=True)
    say(f"[mxfp8 bwd] workload 5 + dO: B={case.batch} tokens={case.total_q}")
    w = bench.Workload(case)
    w.step()
    torch.cuda.synchronize()
    assert w.status.cpu().tolist()[0] == 0
    idx = chosen_samples(case, extra=2)
    say(f"[mxfp8 bwd] workload 5: oracle on samples {idx}")
    qo = np.concatenate([[0], np.cumsum(case.q_lens.astype(np.int64))])
    qr = torch.as_tensor(rows(qo, idx))
    deq = [_dequant(c.cpu()[qr], s.cpu()[qr]) for c, s in
           ((w.qc, w.qs), (w.kc, w.ks), (w.vc, w.vs), (w.doc, w.dos))]
    lens = case.q_lens[idx]
    dq_ref, dk_ref, dv_ref = oracle.backward(deq[0], deq[1], deq[2], deq[3], lens, lens,
                                             causal=True)
    c = oracle.abs_terms(deq[0], deq[1], deq[2], deq[3], lens, lens, causal=True)
    _check("dQ", w.dq.cpu()[qr], dq_ref, c["dQ"])
    _check("dK", w.dk.cpu()[qr], dk_ref, c["dK"])
    _check("dV", w.dv.cpu()[qr], dv_ref, c["dV"])
    for t in (w.dq, w.dk, w.dv):
        assert torch.isfinite(t.float()).all()
