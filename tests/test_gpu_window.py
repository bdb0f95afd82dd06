"""GPU parity for sliding-window attention (jfa_problem.window).

A window W keeps key j for query i only when |i + (kv_len - q_len) - j| < W ("GEM Training: How
Meta Doubled the Efficiency of Its LLM-Scale Ads Foundation Model", "Challenge 1": long
sequences with a short attention window; "Meta Enhances GEM Training Efficiency ...",
"Leveraging Compute Efficiency through Customized Kernels": attention over windows).  The tile
lists must match the oracle's bit for bit, and the forward, backward and bias gradient must
match the oracle within the bf16 bounds (tests/gpu_helpers.py), for windows narrower than a
tile, spanning several tiles and wider than every sample, with and without causal masking."""
import numpy as np
import pytest
import torch

import oracle
from jfa_synth import custom_case
from tests.gpu_helpers import compare, compare_lse, device_case, say
from tests.test_gpu_bias_grad import _check_table, check_dense

pytestmark = pytest.mark.gpu

LENS_Q = [700, 0, 129, 64, 1500, 5, 300]
LENS_KV_ASYM = [500, 40, 200, 64, 1400, 9, 0]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import jagged_attention_amd as jfa
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    jfa.load()
    oracle.build()
    return jfa


@pytest.mark.parametrize("window", [1, 5, 64, 200, 5000])
@pytest.mark.parametrize("causal,asym", [(True, False), (False, False), (False, True),
                                         (True, True)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_window_schedule_bitexact(window, causal, asym, dtype):
    import jagged_attention_amd as jfa
    ql = np.array(LENS_Q, np.int32)
    kl = np.array(LENS_KV_ASYM if asym else LENS_Q, np.int32)
    H = 2
    for slots in (0, 16):
        p = jfa.make_problem(len(ql), H, 128 if dtype == "bf16" else 64, int(ql.sum()),
                             int(kl.sum()), dtype=dtype, causal=causal, split_slots=slots,
                             window=window)
        tc = jfa.jfa_tile_config(p)
        qo = torch.as_tensor(oracle.offsets(ql).astype(np.int32)).cuda()
        ko = torch.as_tensor(oracle.offsets(kl).astype(np.int32)).cuda()
        got = jfa.build_schedule(p, qo, ko)
        want = oracle.schedule(oracle.offsets(ql), oracle.offsets(kl), H, causal, bm=tc["bm"],
                               bn=tc["bn"], slots=tc["slots"], bq_bm=tc["bq_bm"],
                               bq_bn=tc["bq_bn"], bk_bn=tc["bk_bn"], bk_bm=tc["bk_bm"],
                               fuse=int(tc["fuse"]), window=window)
        assert got["status"] == 0
        for key in ("fwd", "fwd_slot", "combine", "bwd_q", "bwd_kv"):
            assert np.array_equal(got[key].numpy(), want[key]), (key, slots)
        assert got["split_threshold"] == want["split_threshold"]


def _run(case, window, split_slots=0):
    import jagged_attention_amd as jfa
    dc = device_case(case)
    kw = dict(mode=case.mode, causal=case.causal, bias=dc["bias"], bias_kind=case.bias_kind,
              num_buckets=case.num_buckets, window=window)
    o, lse = jfa.forward(dc["q"], dc["k"], dc["v"], dc["qo"], dc["ko"], split_slots=split_slots,
                         **kw)
    dq, dk, dv = jfa.backward(dc["q"], dc["k"], dc["v"], o, lse, dc["dout"], dc["qo"], dc["ko"],
                              **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.case_forward(case, window=window)
    dq_ref, dk_ref, dv_ref = oracle.case_backward(case, window=window)
    c = oracle.case_abs_terms(case, window=window)
    compare("O", o, o_ref, case.dtype, cond=c["O"])
    compare_lse(lse, lse_ref, case.mode)
    compare("dQ", dq, dq_ref, case.dtype, cond=c["dQ"])
    compare("dK", dk, dk_ref, case.dtype, cond=c["dK"])
    compare("dV", dv, dv_ref, case.dtype, cond=c["dV"])
    return dc, o


@pytest.mark.parametrize("window", [5, 100, 300])
@pytest.mark.parametrize("mode,causal,bias_kind", [("softmax", True, "relpos"),
                                                    ("softmax", False, "none"),
                                                    ("silu", False, "dense"),
                                                    ("gelu", True, "none")])
@pytest.mark.parametrize("d", [128, 64])
def test_window_parity(window, mode, causal, bias_kind, d):
    """Windows narrower than a 64-key step, spanning two query tiles, and several tiles."""
    kl = LENS_Q if causal else LENS_KV_ASYM
    case = custom_case(LENS_Q, kl, 2, d, dtype="bf16", mode=mode, causal=causal,
                       bias_kind=bias_kind, seed=170 + d)
    say(f"[window] W={window} mode={mode} causal={causal} bias={bias_kind} d={d}")
    _run(case, window)


@pytest.mark.parametrize("window", [1, 64, 10000])
def test_window_edges(window):
    """A window of one key (each query sees only its aligned key), exactly one step, and wider
    than every sample (then equal to full attention); split tiles and fp32 too."""
    case = custom_case(LENS_Q, LENS_Q, 2, 128, dtype="bf16", mode="softmax", causal=True,
                       bias_kind="relpos", seed=180)
    say(f"[window] edges W={window}")
    _run(case, window, split_slots=16)
    case32 = custom_case([130, 0, 77, 64], [130, 0, 77, 64], 2, 64, dtype="f32",
                         mode="gelu", causal=False, bias_kind="dense", seed=181)
    _run(case32, window)


@pytest.mark.parametrize("bias_kind", ["relpos", "dense"])
def test_window_bias_gradient(bias_kind):
    import jagged_attention_amd as jfa
    case = custom_case(LENS_Q, LENS_Q, 2, 128, dtype="bf16", mode="softmax", causal=True,
                       bias_kind=bias_kind, seed=182)
    W = 100
    say(f"[window] dbias W={W} bias={bias_kind}")
    dc = device_case(case)
    kw = dict(mode="softmax", causal=True, bias_kind=bias_kind, num_buckets=case.num_buckets,
              window=W)
    o, lse = jfa.forward(dc["q"], dc["k"], dc["v"], dc["qo"], dc["ko"], bias=dc["bias"], **kw)
    dq, dk, dv, db = jfa.backward_dbias(dc["q"], dc["k"], dc["v"], o, lse, dc["dout"], dc["qo"],
                                        dc["ko"], dc["bias"], **kw)
    torch.cuda.synchronize()
    okw = dict(mode="softmax", causal=True, bias=case.bias, bias_kind=bias_kind,
               num_buckets=case.num_buckets, window=W)
    db_ref = oracle.bias_grad(case.q, case.k, case.v, case.dout, case.q_lens, case.kv_lens,
                              **okw)
    if bias_kind == "dense":
        o_ref, _ = oracle.case_forward(case, window=W)
        do = case.dout.double().numpy()
        resid = np.abs(np.einsum("rhd,rhd->rh", do, o.double().cpu().numpy() - o_ref))
        check_dense(db, db_ref, case, resid)
    else:
        _check_table(db, db_ref)
    dq_ref, dk_ref, dv_ref = oracle.backward(case.q, case.k, case.v, case.dout, case.q_lens,
                                             case.kv_lens, **okw)
    compare("dQ", dq, dq_ref, "bf16")
    compare("dK", dk, dk_ref, "bf16")
    compare("dV", dv, dv_ref, "bf16")

