"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

Each of the five workloads is drawn at its full size and run through the same
``bench.Workload`` the benchmark times (offsets, scheduler, forward, backward, and for
MXFP8 the quantiser, all through the C ABI).  Samples are independent, so the oracle is run
on a sub-batch of chosen samples (the longest, the shortest, empty ones and a seeded random
few) and compared element by element with those samples' rows of the full-size GPU result.
Properties that hold at any size (finite outputs, empty rows exactly zero) are checked on
every row.
"""
import numpy as np
import pytest
import torch

import oracle
from jfa_synth import make_case
from tests.gpu_helpers import compare, compare_lse, say, sub_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import jagged_attention_amd as jfa
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    jfa.load()
    oracle.build()


def chosen_samples(case, extra=3, seed=0):
    n = case.q_lens.astype(np.int64) * np.maximum(case.kv_lens.astype(np.int64), 1)
    idx = {int(np.argmax(n)), int(np.argmin(np.where(case.q_lens > 0, n, n.max() + 1)))}
    idx |= {int(b) for b in np.flatnonzero(case.q_lens == 0)[:2]}
    idx |= {int(b) for b in np.flatnonzero(case.kv_lens == 0)[:2]}
    rng = np.random.default_rng(seed)
    idx |= {int(b) for b in rng.choice(case.batch, size=min(extra, case.batch), replace=False)}
    return sorted(idx)


def rows(offsets, idx):
    return np.concatenate([np.arange(offsets[b], offsets[b + 1]) for b in idx] +
                          [np.zeros(0, np.int64)]).astype(np.int64)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_fullsize_parity(cfg):
    import bench
    case = make_case(cfg)
    say(f"[fullsize] workload {cfg} ({case.name}): B={case.batch} tokens q={case.total_q} "
        f"kv={case.total_kv}")
    w = bench.Workload(case)
    w.step()
    torch.cuda.synchronize()
    assert w.status.cpu().tolist() == [0, 0]
    idx = chosen_samples(case)
    say(f"[fullsize] workload {cfg}: oracle on samples {idx}")
    sub = sub_case(case, idx)
    o_ref, lse_ref = oracle.case_forward(sub)
    dq_ref, dk_ref, dv_ref = oracle.case_backward(sub)
    qo = np.concatenate([[0], np.cumsum(case.q_lens.astype(np.int64))])
    ko = np.concatenate([[0], np.cumsum(case.kv_lens.astype(np.int64))])
    qr = torch.as_tensor(rows(qo, idx))
    kr = torch.as_tensor(rows(ko, idx))
    dt = "f32" if case.dtype == "f32" else "bf16"
    o = w.o.cpu()
    compare("O", o[qr], o_ref, dt)
    if case.mode == "softmax":
        compare_lse(w.lse.cpu()[:, qr], lse_ref, case.mode, tol=1e-5 if dt == "f32" else 1e-3)
    compare("dQ", w.dq.cpu()[qr], dq_ref, dt)
    compare("dK", w.dk.cpu()[kr], dk_ref, dt)
    compare("dV", w.dv.cpu()[kr], dv_ref, dt)
    # every row: finite, and rows of samples without keys are exactly zero
    for t in (w.o, w.dq, w.dk, w.dv):
        assert torch.isfinite(t.float()).all()
    empty_q = rows(qo, np.flatnonzero(case.kv_lens == 0))
    if empty_q.size:
        assert torch.all(o[torch.as_tensor(empty_q)] == 0)


def test_fullsize_mxfp8():
    import bench
    case = make_case(5)
    say(f"[fullsize] workload 5 ({case.name}): B={case.batch} tokens={case.total_q} "
        f"max len={int(case.q_lens.max())}")
    w = bench.Workload(case, with_backward=False)
    w.step()
    torch.cuda.synchronize()
    idx = chosen_samples(case)
    say(f"[fullsize] workload 5: oracle on samples {idx}")
    qo = np.concatenate([[0], np.cumsum(case.q_lens.astype(np.int64))])
    qr = rows(qo, idx)
    qrt = torch.as_tensor(qr)
    deq = []
    for x, c, s in ((case.q, w.qc, w.qs), (case.k, w.kc, w.ks), (case.v, w.vc, w.vs)):
        want_c, want_s = oracle.mxfp8_quantize(x[qrt].double().numpy())
        assert np.array_equal(c.cpu()[qrt].numpy(), want_c)          # quantiser bit-exact
        assert np.array_equal(s.cpu()[qrt].numpy(), want_s)
        deq.append(oracle.mxfp8_dequantize(want_c, want_s))
    lens = case.q_lens[idx]
    o_ref, lse_ref = oracle.forward(deq[0], deq[1], deq[2], lens, lens, causal=True)
    from tests.helpers import rel_l2
    got = w.o.cpu()[qrt].float().numpy()
    rl = rel_l2(got, o_ref)
    say(f"[fullsize] workload 5: O rel-L2 {rl:.3g}")
    assert rl <= 5e-2
    compare_lse(w.lse.cpu()[:, qrt], lse_ref, "softmax", tol=1e-2)
    assert torch.isfinite(w.o.float()).all()
