"""The whole path captured in a HIP graph (torch.cuda.CUDAGraph) and replayed: every replay,
with eager work and synchronisations between replays, must reproduce the eager results bit for
bit (all kernels are deterministic), and the eager results match the oracle."""
import pytest
import torch

import oracle
from jfa_synth import custom_case
from tests.gpu_helpers import compare, say
from tests.test_gpu_bias_grad import check_dense, d_residue

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import jagged_attention_amd as jfa
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    jfa.load()
    oracle.build()
    return jfa


@pytest.mark.parametrize("mode,causal,bias_kind,split", [("softmax", True, "relpos", 4),
                                                          ("gelu", False, "dense", 0)])
def test_graph_replay_matches_eager(mode, causal, bias_kind, split):
    import jagged_attention_amd as jfa
    lens = [700, 0, 129, 64, 1500]
    kl = lens if causal else [300, 16, 64, 1, 90]
    case = custom_case(lens, kl, 2, 128, dtype="bf16", mode=mode, causal=causal,
                       bias_kind=bias_kind, seed=77)
    say(f"[graph] mode={mode} causal={causal} bias={bias_kind} split={split}")
    dev = torch.device("cuda:0")
    ql = torch.as_tensor(case.q_lens, dtype=torch.int32, device=dev)
    kvl = torch.as_tensor(case.kv_lens, dtype=torch.int32, device=dev)
    q, k, v, do = (t.to(dev).contiguous() for t in (case.q, case.k, case.v, case.dout))
    bias = None if case.bias is None else case.bias.to(dev).contiguous()
    B, H, d = case.batch, case.heads, case.head_dim
    pf = jfa.make_problem(B, H, d, case.total_q, case.total_kv, mode=mode, causal=causal,
                          bias_kind=bias_kind, split_slots=split)
    pb = jfa.make_problem(B, H, d, case.total_q, case.total_kv, mode=mode, causal=causal,
                          bias_kind=bias_kind)
    wf = torch.empty(jfa.jfa_workspace_bytes(pf, False), dtype=torch.uint8, device=dev)
    wb = torch.empty(jfa.jfa_workspace_bytes(pb, True), dtype=torch.uint8, device=dev)
    qo = torch.empty(B + 1, dtype=torch.int32, device=dev)
    ko = torch.empty(B + 1, dtype=torch.int32, device=dev)
    st = torch.zeros(2, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((H, case.total_q), dtype=torch.float32, device=dev) \
        if mode == "softmax" else None
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def step():
        jfa.jfa_lengths_to_offsets(ql, B, qo, status=st[0:1])
        jfa.jfa_lengths_to_offsets(kvl, B, ko, status=st[1:2])
        jfa.jfa_forward(pf, q, k, v, None, None, None, qo, ko, bias, o, lse, wf, wf.numel())
        jfa.jfa_backward(pb, q, k, v, o, lse, do, qo, ko, bias, dq, dk, dv, wb, wb.numel())

    outs = [o, dq, dk, dv] + ([lse] if lse is not None else [])
    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    o_ref, _ = oracle.case_forward(case)
    dq_ref, dk_ref, dv_ref = oracle.case_backward(case)
    c = oracle.case_abs_terms(case)     # bf16 operand rounding (one sample has a single key)
    for name, got, ref in (("O", o, o_ref), ("dQ", dq, dq_ref), ("dK", dk, dk_ref),
                           ("dV", dv, dv_ref)):
        compare(name, got, ref, "bf16", cond=c[name])

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = custom_case([33, 90], [33, 90], 2, 128, dtype="bf16", seed=5, with_dout=False)
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        # eager work of the program between replays
        oq = other.q.to(dev)
        qo2, _ = jfa.lengths_to_offsets(torch.as_tensor(other.q_lens, dtype=torch.int32,
                                                        device=dev))
        jfa.forward(oq, other.k.to(dev), other.v.to(dev), qo2, qo2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, want):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        assert int(st[0].item()) == 0 and int(st[1].item()) == 0


@pytest.mark.parametrize("bias_kind", ["relpos", "dense"])
def test_graph_replay_bias_gradient(bias_kind):
    """jfa_backward_dbias inside a captured graph: its zeroing is a fill kernel (no memset node),
    so every replay, with eager library work in between, reproduces the eager dQ, dK, dV and
    dbias bit for bit, after each output was filled with NaN."""
    import jagged_attention_amd as jfa
    lens = [700, 0, 129, 64, 1500]
    case = custom_case(lens, lens, 2, 128, dtype="bf16", mode="softmax", causal=True,
                       bias_kind=bias_kind, seed=78)
    say(f"[graph dbias] bias={bias_kind}")
    dev = torch.device("cuda:0")
    ql = torch.as_tensor(case.q_lens, dtype=torch.int32, device=dev)
    q, k, v, do = (t.to(dev).contiguous() for t in (case.q, case.k, case.v, case.dout))
    bias = case.bias.to(dev).contiguous()
    B, H, d = case.batch, case.heads, case.head_dim
    p = jfa.make_problem(B, H, d, case.total_q, case.total_kv, mode="softmax", causal=True,
                         bias_kind=bias_kind)
    wf = torch.empty(jfa.jfa_workspace_bytes(p, 0), dtype=torch.uint8, device=dev)
    wb = torch.empty(jfa.jfa_workspace_bytes(p, 2), dtype=torch.uint8, device=dev)
    qo = torch.empty(B + 1, dtype=torch.int32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((H, case.total_q), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    db = torch.empty_like(bias)

    def step():
        jfa.jfa_lengths_to_offsets(ql, B, qo, status=st[0:1])
        jfa.jfa_forward(p, q, k, v, None, None, None, qo, qo, bias, o, lse, wf, wf.numel())
        jfa.jfa_backward_dbias(p, q, k, v, o, lse, do, qo, qo, bias, dq, dk, dv, db, wb,
                               wb.numel())

    outs = [o, lse, dq, dk, dv, db]
    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    db_ref = oracle.bias_grad(case.q, case.k, case.v, case.dout, case.q_lens, case.kv_lens,
                              mode="softmax", causal=True, bias=case.bias, bias_kind=bias_kind)
    if bias_kind == "dense":
        check_dense(db, db_ref, case, d_residue(case, o))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = custom_case([33, 90], [33, 90], 2, 128, dtype="bf16", seed=5, with_dout=False)
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        oq = other.q.to(dev)
        qo2, _ = jfa.lengths_to_offsets(torch.as_tensor(other.q_lens, dtype=torch.int32,
                                                        device=dev))
        jfa.forward(oq, other.k.to(dev), other.v.to(dev), qo2, qo2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, want):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
