"""GPU parity for the bias gradient (jfa_backward_dbias) against the oracle's ``bias_grad``.

The bias is a trained parameter ("Meta GEM Training Efficiency: ...", section "Bottleneck
move 1": custom biases), so the backward also returns dL/dbias: per pair for a dense bias (bf16,
in the bias's layout), summed by bucket for the relative-position table (fp32 [H, buckets]).

Bounds: the dense gradient is bf16 per pair, so the bf16 bounds apply as for dQ/dK/dV.  A table
entry sums dS over up to a few hundred thousand pairs; its error scales with the magnitude of
the sum, so the max-abs bound is 2e-2 * max(1, max |exact|), with rel-L2 1e-2 as for bf16.
"""
import numpy as np
import pytest
import torch

import oracle
from jfa_synth import custom_case
from tests.gpu_helpers import bf16_half_ulp, compare, device_case, say
from tests.helpers import max_abs, rel_l2

pytestmark = pytest.mark.gpu

LENS_Q = [300, 17, 129, 0, 64, 700, 5]
LENS_KV = [300, 40, 129, 9, 0, 700, 200]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import jagged_attention_amd as jfa
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    jfa.load()
    oracle.build()
    return jfa


def _run(case, dc, with_o=False):
    import jagged_attention_amd as jfa
    kw = dict(mode=case.mode, causal=case.causal, bias_kind=case.bias_kind,
              num_buckets=case.num_buckets)
    o, lse = jfa.forward(dc["q"], dc["k"], dc["v"], dc["qo"], dc["ko"], bias=dc["bias"], **kw)
    out = jfa.backward_dbias(dc["q"], dc["k"], dc["v"], o, lse, dc["dout"], dc["qo"], dc["ko"],
                             dc["bias"], **kw)
    torch.cuda.synchronize()
    return (out, o) if with_o else out


def d_residue(case, o_gpu, bias=None, num_buckets=None):
    """Softmax: |dO_i . (O_i - O_bf16,i)| per (query row, head). The backward forms
    D = rowsum(dO * O) from the stored bf16 O, and a pair's dS = P (dP - D) carries P times this
    (P <= 1); 0 for GDPA, which has no D."""
    if case.mode != "softmax":
        return np.zeros((case.total_q, case.heads))
    o_ref, _ = oracle.forward(case.q, case.k, case.v, case.q_lens, case.kv_lens, mode="softmax",
                              causal=case.causal, bias=case.bias if bias is None else bias,
                              bias_kind=case.bias_kind,
                              num_buckets=num_buckets or case.num_buckets)
    do = case.dout.double().numpy()
    return np.abs(np.einsum("rhd,rhd->rh", do, o_gpu.double().cpu().numpy() - o_ref))


def check_dense(db, ref, case, resid):
    """Dense dbias against the oracle: element-wise |got - exact| <= 2e-2 + half a bf16 ulp of
    the exact value + the pair's row residue (d_residue), and rel-L2 <= 1e-2."""
    H = case.heads
    slack = []
    qo = 0
    for n, m in zip(case.q_lens, case.kv_lens):
        n, m = int(n), int(m)
        for h in range(H):
            slack.append(np.repeat(resid[qo:qo + n, h], m))
        qo += n
    slack = np.concatenate(slack) if slack else np.zeros(0)
    g = db.detach().float().cpu().double().numpy()
    assert slack.shape == g.shape == ref.shape
    err = np.abs(g - ref) - bf16_half_ulp(ref) - slack
    rl = rel_l2(g, ref)
    say(f"  dense dbias: max-abs {max_abs(g, ref):.3e}, beyond rounding and D residue "
        f"{err.max():.3e}, rel-L2 {rl:.3e}")
    assert np.all(np.isfinite(g)) and err.max() <= 2e-2 and rl <= 1e-2


def _check_table(got, want):
    g = got.detach().double().cpu().numpy()
    ma, rl = max_abs(g, want), rel_l2(g, want)
    bound = 2e-2 * max(1.0, float(np.abs(want).max()))
    say(f"  dbias table: max-abs {ma:.3e} (bound {bound:.3e}) rel-L2 {rl:.3e}")
    assert ma <= bound and rl <= 1e-2


@pytest.mark.parametrize("mode", ["softmax", "silu", "gelu"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("bias_kind", ["relpos", "dense"])
@pytest.mark.parametrize("d", [128, 64])
def test_bias_grad_parity(mode, causal, bias_kind, d):
    lq, lk = (LENS_Q, LENS_Q) if causal else (LENS_Q, LENS_KV)
    case = custom_case(lq, lk, 2, d, dtype="bf16", mode=mode, causal=causal,
                       bias_kind=bias_kind, seed=90 + d)
    say(f"[bias grad] mode={mode} causal={causal} bias={bias_kind} d={d}")
    dc = device_case(case)
    (dq, dk, dv, db), o = _run(case, dc, with_o=True)
    okw = dict(mode=mode, causal=causal, bias=case.bias, bias_kind=bias_kind,
               num_buckets=case.num_buckets)
    db_ref = oracle.bias_grad(case.q, case.k, case.v, case.dout, case.q_lens, case.kv_lens,
                              **okw)
    if bias_kind == "dense":
        assert db.dtype == torch.bfloat16 and db.shape == dc["bias"].shape
        check_dense(db, db_ref, case, d_residue(case, o))
    else:
        assert db.dtype == torch.float32 and tuple(db.shape) == (2, case.num_buckets)
        _check_table(db, db_ref)
    dq_ref, dk_ref, dv_ref = oracle.backward(case.q, case.k, case.v, case.dout, case.q_lens,
                                             case.kv_lens, **okw)
    compare("dQ", dq, dq_ref, "bf16")
    compare("dK", dk, dk_ref, "bf16")
    compare("dV", dv, dv_ref, "bf16")


@pytest.mark.parametrize("num_buckets", [1, 17, 64, 65, 300, 1500])
@pytest.mark.parametrize("causal", [True, False])
def test_bias_grad_table_widths(num_buckets, causal):
    """Tables of at most 64 buckets are summed in LDS, wider ones in memory (two lane halves per
    row); both against the oracle, with the two-stage reduction over a few thousand rows."""
    lens = [1500, 3, 700, 64, 2000, 129]
    case = custom_case(lens, lens, 3, 64, dtype="bf16", mode="gelu" if causal else "softmax",
                       causal=causal, bias_kind="relpos", num_buckets=num_buckets, seed=11)
    say(f"[bias grad table] buckets={num_buckets} causal={causal}")
    dc = device_case(case)
    out, o = _run(case, dc, with_o=True)
    db = out[3]
    db_ref = oracle.bias_grad(case.q, case.k, case.v, case.dout, case.q_lens, case.kv_lens,
                              mode=case.mode, causal=causal, bias=case.bias, bias_kind="relpos",
                              num_buckets=num_buckets)
    assert tuple(db.shape) == (3, num_buckets)
    if case.mode == "softmax" and num_buckets == 1:
        # one bucket under softmax: a constant added to a whole row leaves the output alone, so
        # the exact gradient is 0; what remains is the backward's D = rowsum(dO * O) taken from
        # the stored bf16 O, |sum over the row's pairs of P (D_exact - D)| = |dO . (O - O_bf16)|
        # per row, which bounds the sum over rows
        o_ref, _ = oracle.forward(case.q, case.k, case.v, case.q_lens, case.kv_lens,
                                  mode="softmax", causal=causal, bias=case.bias,
                                  bias_kind="relpos", num_buckets=1)
        do = case.dout.double().numpy()
        resid = np.abs(np.einsum("rhd,rhd->rh", do, o.double().cpu().numpy() - o_ref))
        bound = resid.sum(axis=0) * 1.05 + 1e-3
        got = np.abs(db.double().cpu().numpy()[:, 0])
        say(f"  one bucket: |dbias| {got} bound {bound} (exact {db_ref[:, 0]})")
        assert np.all(np.abs(db_ref) < 1e-9) and np.all(got <= bound)
        return
    _check_table(db, db_ref)


@pytest.mark.parametrize("bias_kind", ["relpos", "dense"])
def test_bias_grad_deterministic_and_overwrites(bias_kind):
    """Two calls give bitwise-identical results, whatever the output buffer held before."""
    import jagged_attention_amd as jfa
    case = custom_case(LENS_Q, LENS_Q, 2, 128, dtype="bf16", mode="softmax", causal=True,
                       bias_kind=bias_kind, seed=7)
    say(f"[bias grad determinism] bias={bias_kind}")
    dc = device_case(case)
    a = _run(case, dc)
    b = _run(case, dc)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)
    # the dense gradient is zero on every pair that is not visible (here: above the diagonal);
    # the mask comes from the indices, since a visible pair's exact dS can be 0 as well (a row
    # with one visible key has P = 1 and dS = dP - D = 0)
    if bias_kind == "dense":
        db = a[3].float().cpu().numpy()
        hidden = []
        for n in LENS_Q:
            i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
            hidden.append(np.tile((j > i).ravel(), 2))
        hidden = np.concatenate(hidden)
        assert hidden.shape == db.shape and hidden.sum() > 0
        assert np.all(db[hidden] == 0)


def test_bias_grad_rejects_unsupported():
    import jagged_attention_amd as jfa
    case = custom_case([64], [64], 1, 64, dtype="f32", mode="softmax", bias_kind="relpos", seed=3)
    dc = device_case(case)
    o, lse = jfa.forward(dc["q"], dc["k"], dc["v"], dc["qo"], dc["ko"], bias=dc["bias"],
                         bias_kind="relpos")
    with pytest.raises(jfa.JfaError):
        jfa.backward_dbias(dc["q"], dc["k"], dc["v"], o, lse, dc["dout"], dc["qo"], dc["ko"],
                           dc["bias"], bias_kind="relpos")


@pytest.mark.parametrize("bias_kind", ["relpos", "dense"])
def test_bias_grad_block_attention(bias_kind):
    """The bias gradient of BlockAttention: the library's refined offsets in front of
    jfa_backward_dbias, against the oracle's block-diagonal bias gradient on the original
    samples (a dense bias is laid out over the blocks)."""
    import jagged_attention_amd as jfa
    lens = [300, 17, 129, 0, 64, 700]
    w = 100
    case = custom_case(lens, lens, 2, 128, dtype="bf16", mode="silu", causal=True,
                       bias_kind="relpos", seed=61)
    say(f"[bias grad block attention] bias={bias_kind} w={w}")
    dc = device_case(case)
    boff, nb, st = jfa.block_offsets(dc["qo"], w, case.total_q)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    blocks = [min(w, n - s) for n in lens for s in range(0, n, w)]
    if bias_kind == "dense":
        g = torch.Generator().manual_seed(62)
        bias = (0.1 * torch.randn(2 * sum(b * b for b in blocks), generator=g)).to(torch.bfloat16)
    else:
        bias = case.bias
    kw = dict(mode="silu", causal=True, bias_kind=bias_kind, num_buckets=case.num_buckets)
    bd = bias.cuda()
    o, lse = jfa.forward(dc["q"], dc["k"], dc["v"], boff, boff, bias=bd, **kw)
    dq, dk, dv, db = jfa.backward_dbias(dc["q"], dc["k"], dc["v"], o, lse, dc["dout"], boff,
                                        boff, bd, **kw)
    torch.cuda.synchronize()
    if bias_kind == "dense":
        # the oracle's dense layout is per sample; over the blocks taken as samples it is the
        # refined batch's layout
        bl = np.array(blocks)
        ref = oracle.bias_grad(case.q, case.k, case.v, case.dout, bl, bl, mode="silu",
                               causal=True, bias=bias, bias_kind="dense")
        compare("dbias", db, ref, "bf16")
    else:
        ref = oracle.bias_grad(case.q, case.k, case.v, case.dout, case.q_lens, case.kv_lens,
                               mode="silu", causal=True, bias=bias, bias_kind="relpos",
                               num_buckets=case.num_buckets, block=w)
        _check_table(db, ref)
        dq_ref, dk_ref, _ = oracle.backward(case.q, case.k, case.v, case.dout, case.q_lens,
                                            case.kv_lens, mode="silu", causal=True,
                                            bias=bias, bias_kind="relpos",
                                            num_buckets=case.num_buckets, block=w)
        compare("dQ", dq, dq_ref, "bf16")
        compare("dK", dk, dk_ref, "bf16")


@pytest.mark.parametrize("mode,causal,bias_kind", [("softmax", True, "relpos"),
                                                    ("gelu", False, "dense")])
def test_autograd_bias_gradient(mode, causal, bias_kind):
    """A trainable bias through the torch.autograd.Function: bias.grad is the oracle's
    dL/dbias for L = <O, dO>, beside dQ, dK, dV."""
    import jagged_attention_amd as jfa
    lq = [150, 0, 70, 9]
    lk = lq if causal else [90, 12, 130, 3]
    case = custom_case(lq, lk, 2, 128, dtype="bf16", mode=mode, causal=causal,
                       bias_kind=bias_kind, seed=96)
    say(f"[bias grad] autograd mode={mode} bias={bias_kind}")
    dc = device_case(case)
    q, k, v = (dc[x].clone().requires_grad_(True) for x in ("q", "k", "v"))
    bias = dc["bias"].clone().requires_grad_(True)
    opts = dict(mode=mode, causal=causal, bias_kind=bias_kind, num_buckets=case.num_buckets)
    o = jfa.JaggedAttention.apply(q, k, v, dc["qo"], dc["ko"], bias, opts)
    (o.float() * dc["dout"].float()).sum().backward()
    torch.cuda.synchronize()
    okw = dict(mode=mode, causal=causal, bias=case.bias, bias_kind=bias_kind,
               num_buckets=case.num_buckets)
    db_ref = oracle.bias_grad(case.q, case.k, case.v, case.dout, case.q_lens, case.kv_lens,
                              **okw)
    assert bias.grad is not None and bias.grad.dtype == bias.dtype
    if bias_kind == "dense":
        check_dense(bias.grad, db_ref, case, d_residue(case, o.detach()))
    else:
        _check_table(bias.grad, db_ref)
    dq_ref, dk_ref, dv_ref = oracle.backward(case.q, case.k, case.v, case.dout, case.q_lens,
                                             case.kv_lens, **okw)
    compare("dQ", q.grad, dq_ref, "bf16")
    compare("dK", k.grad, dk_ref, "bf16")
    compare("dV", v.grad, dv_ref, "bf16")


def test_malformed_offsets_leave_dbias_untouched():
    """Offsets the scheduler rejects (non-monotone) on a workspace and dbias prefilled with
    garbage: the call reports JFA_ERR_DEVICE_DATA and writes neither dbias nor the gradients
    (the zeroing kernel takes its count from bias offsets that were never written)."""
    import jagged_attention_amd as jfa
    for bias_kind in ("dense", "relpos"):
        case = custom_case([40, 30], [40, 30], 2, 128, dtype="bf16", mode="softmax",
                           causal=True, bias_kind=bias_kind, seed=97)
        say(f"[bias grad] malformed offsets bias={bias_kind}")
        dc = device_case(case)
        bad = torch.tensor([0, 50, 30], dtype=torch.int32, device="cuda:0")   # decreasing
        p = jfa.make_problem(2, 2, 128, case.total_q, case.total_kv, mode="softmax",
                             causal=True, bias_kind=bias_kind)
        nb = jfa.jfa_workspace_bytes(p, 2)
        ws = torch.full((nb,), 0x7F, dtype=torch.uint8, device="cuda:0")
        o = torch.zeros_like(dc["q"])
        lse = torch.zeros((2, case.total_q), dtype=torch.float32, device="cuda:0")
        dq, dk, dv = (torch.full_like(dc[x], 3.0) for x in ("q", "k", "v"))
        db = torch.full_like(dc["bias"], 5.0)
        jfa.jfa_backward_dbias(p, dc["q"], dc["k"], dc["v"], o, lse, dc["dout"], bad, bad,
                               dc["bias"], dq, dk, dv, db, ws, nb)
        assert jfa.jfa_read_device_status(ws) == jfa._lib.JFA_ERR_DEVICE_DATA
        assert bool((db == 5.0).all()), bias_kind
        assert bool((dq == 3.0).all() and (dk == 3.0).all() and (dv == 3.0).all())
