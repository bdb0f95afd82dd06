"""CPU-side checks of the C ABI: the library loads, exports every declared symbol, and rejects
bad arguments on the host before anything is enqueued (no GPU needed, no compute calls)."""
import ctypes
import os
import re

import pytest

import jagged_attention_amd as jfa
from jagged_attention_amd import _lib
from tests.conftest import ROOT

FAKE = 0x10000          # never dereferenced: every call below fails host validation first


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "jfa.h")).read()
    return sorted(set(re.findall(r"\b(jfa_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_are_exported():
    lib = jfa.load()
    declared = _declared_symbols()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(_lib.EXPORTS) == declared


def test_status_strings():
    for code, name in ((0, "JFA_OK"), (-1, "JFA_ERR_INVALID_ARG"), (-2, "JFA_ERR_UNSUPPORTED"),
                       (-3, "JFA_ERR_WORKSPACE"), (-4, "JFA_ERR_LAUNCH"),
                       (-5, "JFA_ERR_DEVICE_DATA")):
        assert _lib.status_string(code) == name


def _problem(**kw):
    args = dict(batch=4, heads=2, head_dim=128, total_q=1000, total_kv=900, split_slots=64)
    args.update(kw)
    b, h, d, tq, tk = (args.pop(k) for k in ("batch", "heads", "head_dim", "total_q", "total_kv"))
    return jfa.make_problem(b, h, d, tq, tk, **args)


def test_negative_window_is_invalid():
    p = _problem(window=-1)
    assert jfa.jfa_workspace_bytes(p, False) == 0
    assert jfa.load().jfa_tile_config(ctypes.byref(p), (ctypes.c_int32 * 8)()) == \
        _lib.JFA_ERR_INVALID_ARG
    assert jfa.jfa_workspace_bytes(_problem(window=7), False) > 0


def test_tile_config_and_workspace_host_only():
    p = _problem()
    tc = jfa.jfa_tile_config(p)
    assert tc["bm"] in (64, 128) and tc["bn"] == 64 and tc["slots"] == 64
    assert jfa.jfa_workspace_bytes(p, False) > 0
    assert jfa.jfa_workspace_bytes(p, True) > 0
    short = _problem(batch=100, total_q=3000, total_kv=20000)    # mean q length 30
    assert jfa.jfa_tile_config(short)["bm"] == 64
    f32 = _problem(dtype="f32")
    tc = jfa.jfa_tile_config(f32)
    assert tc["slots"] == -1 and tc["bm"] == 64


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), _lib.JFA_ERR_UNSUPPORTED),
    (dict(batch=0), _lib.JFA_ERR_INVALID_ARG),
    (dict(heads=0), _lib.JFA_ERR_INVALID_ARG),
    (dict(total_q=-1), _lib.JFA_ERR_INVALID_ARG),
    (dict(kv_len_normalize=1), _lib.JFA_ERR_INVALID_ARG),          # softmax cannot normalise
    (dict(bias_kind="relpos", num_buckets=0), _lib.JFA_ERR_INVALID_ARG),
    (dict(total_q=2 ** 31), _lib.JFA_ERR_INVALID_ARG),
])
def test_problem_validation(kw, status):
    p = _problem(**kw)
    with pytest.raises(_lib.JfaError) as e:
        jfa.jfa_tile_config(p)
    assert e.value.status == status
    assert jfa.jfa_workspace_bytes(p, False) == 0


def test_bad_enum_values():
    p = _problem()
    p.mode = 7
    with pytest.raises(_lib.JfaError) as e:
        jfa.jfa_tile_config(p)
    assert e.value.status == _lib.JFA_ERR_INVALID_ARG
    p = _problem()
    p.causal = 2
    assert jfa.jfa_workspace_bytes(p, True) == 0


def _fwd(p, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, qs=None, ks=None, vs=None, qo=FAKE, ko=FAKE, bias=None,
                o=FAKE, lse=FAKE, ws=FAKE, nbytes=1 << 40)
    args.update(over)
    return jfa.load().jfa_forward(ctypes.byref(p), args["q"], args["k"], args["v"], args["qs"],
                                  args["ks"], args["vs"], args["qo"], args["ko"], args["bias"],
                                  args["o"], args["lse"], args["ws"], args["nbytes"], None)


def _bwd(p, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, qo=FAKE, ko=FAKE, bias=None,
                dq=FAKE, dk=FAKE, dv=FAKE, ws=FAKE, nbytes=1 << 40)
    args.update(over)
    return jfa.load().jfa_backward(ctypes.byref(p), args["q"], args["k"], args["v"], args["o"],
                                   args["lse"], args["do"], args["qo"], args["ko"], args["bias"],
                                   args["dq"], args["dk"], args["dv"], args["ws"], args["nbytes"],
                                   None)


def test_forward_host_errors():
    p = _problem()
    assert _fwd(p, q=None) == _lib.JFA_ERR_INVALID_ARG
    assert _fwd(p, o=None) == _lib.JFA_ERR_INVALID_ARG
    assert _fwd(p, lse=None) == _lib.JFA_ERR_INVALID_ARG            # softmax needs LSE
    assert _fwd(p, q=FAKE + 2) == _lib.JFA_ERR_INVALID_ARG          # misaligned
    assert _fwd(p, ws=FAKE + 16) == _lib.JFA_ERR_INVALID_ARG        # workspace not 256-aligned
    assert _fwd(p, bias=FAKE) == _lib.JFA_ERR_INVALID_ARG           # bias without a bias kind
    assert _fwd(p, nbytes=16) == _lib.JFA_ERR_WORKSPACE
    pb = _problem(bias_kind="dense")
    assert _fwd(pb) == _lib.JFA_ERR_INVALID_ARG                      # bias kind without bias
    p8 = _problem(dtype="mxfp8")
    assert _fwd(p8) == _lib.JFA_ERR_INVALID_ARG                      # scales missing
    assert _fwd(p8, qs=FAKE, ks=FAKE, vs=FAKE, nbytes=16) == _lib.JFA_ERR_WORKSPACE
    g = _problem(mode="gelu")
    assert _fwd(g, lse=None, nbytes=16) == _lib.JFA_ERR_WORKSPACE    # GDPA needs no LSE


def test_backward_host_errors():
    p = _problem()
    assert _bwd(p, dq=None) == _lib.JFA_ERR_INVALID_ARG
    assert _bwd(p, lse=None) == _lib.JFA_ERR_INVALID_ARG
    assert _bwd(p, o=None) == _lib.JFA_ERR_INVALID_ARG
    assert _bwd(p, dk=FAKE + 8) == _lib.JFA_ERR_INVALID_ARG
    assert _bwd(p, nbytes=16) == _lib.JFA_ERR_WORKSPACE
    assert _bwd(_problem(dtype="mxfp8")) == _lib.JFA_ERR_UNSUPPORTED
    g = _problem(mode="silu")
    assert _bwd(g, o=None, lse=None, nbytes=16) == _lib.JFA_ERR_WORKSPACE


def test_other_entry_points_host_errors():
    lib = jfa.load()
    assert lib.jfa_lengths_to_offsets(None, 4, FAKE, None, None, None, None) == \
        _lib.JFA_ERR_INVALID_ARG
    assert lib.jfa_lengths_to_offsets(FAKE, -1, FAKE, None, None, None, None) == \
        _lib.JFA_ERR_INVALID_ARG
    # the int64 bias offsets must be 8-byte aligned, the kv lengths 4-byte aligned
    assert lib.jfa_lengths_to_offsets(FAKE, 4, FAKE, FAKE + 4, None, None, None) == \
        _lib.JFA_ERR_INVALID_ARG
    assert lib.jfa_lengths_to_offsets(FAKE, 4, FAKE, FAKE, FAKE + 2, None, None) == \
        _lib.JFA_ERR_INVALID_ARG
    # BlockAttention offsets: block < 1, a negative batch or out_batch, null or misaligned
    assert lib.jfa_block_offsets(FAKE, 4, 0, FAKE, 8, None, None) == _lib.JFA_ERR_INVALID_ARG
    assert lib.jfa_block_offsets(FAKE, -1, 4, FAKE, 8, None, None) == _lib.JFA_ERR_INVALID_ARG
    assert lib.jfa_block_offsets(FAKE, 4, 4, FAKE, -1, None, None) == _lib.JFA_ERR_INVALID_ARG
    assert lib.jfa_block_offsets(None, 4, 4, FAKE, 8, None, None) == _lib.JFA_ERR_INVALID_ARG
    assert lib.jfa_block_offsets(FAKE, 4, 4, FAKE + 2, 8, None, None) == _lib.JFA_ERR_INVALID_ARG
    assert lib.jfa_quantize_mxfp8(FAKE, 10, 48, FAKE, FAKE, None) == _lib.JFA_ERR_INVALID_ARG
    assert lib.jfa_quantize_mxfp8(FAKE + 2, 10, 64, FAKE, FAKE, None) == _lib.JFA_ERR_INVALID_ARG
    # the batched quantiser: 1 to 4 tensors, d % 32 == 0, rows >= 0, aligned non-null pointers
    arr = lambda *v: (ctypes.c_void_p * len(v))(*v)
    rows = lambda *v: (ctypes.c_int64 * len(v))(*v)
    q = lib.jfa_quantize_mxfp8_batch
    assert q(0, arr(FAKE), rows(10), 64, arr(FAKE), arr(FAKE), None) == _lib.JFA_ERR_INVALID_ARG
    assert q(5, arr(*[FAKE] * 5), rows(*[10] * 5), 64, arr(*[FAKE] * 5), arr(*[FAKE] * 5),
             None) == _lib.JFA_ERR_INVALID_ARG
    assert q(2, arr(FAKE, FAKE), rows(10, 10), 48, arr(FAKE, FAKE), arr(FAKE, FAKE), None) == \
        _lib.JFA_ERR_INVALID_ARG
    assert q(2, arr(FAKE, FAKE + 2), rows(10, 10), 64, arr(FAKE, FAKE), arr(FAKE, FAKE),
             None) == _lib.JFA_ERR_INVALID_ARG
    assert q(2, arr(FAKE, FAKE), rows(10, -1), 64, arr(FAKE, FAKE), arr(FAKE, FAKE), None) == \
        _lib.JFA_ERR_INVALID_ARG
    assert q(2, arr(FAKE, None), rows(10, 10), 64, arr(FAKE, FAKE), arr(FAKE, FAKE), None) == \
        _lib.JFA_ERR_INVALID_ARG
    out = ctypes.c_int32(0)
    assert lib.jfa_read_device_status(None, None, ctypes.byref(out)) == _lib.JFA_ERR_INVALID_ARG
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.jfa_kernel_timing(b"", None, ctypes.byref(n)) == _lib.JFA_ERR_INVALID_ARG
    jfa.jfa_kernel_timing_reset()
    assert jfa.jfa_kernel_timing("") == (0.0, 0)


def _bwd_db(p, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, qo=FAKE, ko=FAKE, bias=FAKE,
                dq=FAKE, dk=FAKE, dv=FAKE, db=FAKE, ws=FAKE, nbytes=1 << 40)
    args.update(over)
    return jfa.load().jfa_backward_dbias(ctypes.byref(p), args["q"], args["k"], args["v"],
                                         args["o"], args["lse"], args["do"], args["qo"],
                                         args["ko"], args["bias"], args["dq"], args["dk"],
                                         args["dv"], args["db"], args["ws"], args["nbytes"], None)


def test_backward_dbias_host_errors():
    p = _problem(bias_kind="relpos")
    assert _bwd_db(p, db=None) == _lib.JFA_ERR_INVALID_ARG
    assert _bwd_db(p, bias=None) == _lib.JFA_ERR_INVALID_ARG
    assert _bwd_db(p, db=FAKE + 2) == _lib.JFA_ERR_INVALID_ARG
    assert _bwd_db(_problem(), bias=None) == _lib.JFA_ERR_UNSUPPORTED       # no bias to train
    assert _bwd_db(_problem(bias_kind="relpos", dtype="f32")) == _lib.JFA_ERR_UNSUPPORTED
    # the relative-position table's per-row partials live in the workspace
    assert _bwd_db(p, nbytes=jfa.jfa_workspace_bytes(p, 1)) == _lib.JFA_ERR_WORKSPACE
    assert jfa.jfa_workspace_bytes(p, 2) > jfa.jfa_workspace_bytes(p, 1)
    wide = _problem(bias_kind="relpos", num_buckets=300)     # partial rows per lane half
    assert jfa.jfa_workspace_bytes(wide, 2) > jfa.jfa_workspace_bytes(wide, 1)
    d = _problem(bias_kind="dense")
    assert jfa.jfa_workspace_bytes(d, 2) == jfa.jfa_workspace_bytes(d, 1)
    assert _bwd_db(d, nbytes=16) == _lib.JFA_ERR_WORKSPACE


def test_norm_quant_host_errors():
    lib = jfa.load()
    f = lib.jfa_rmsnorm_quantize_mxfp8
    assert f(FAKE, None, 4, 96, 1e-6, FAKE, FAKE, None) == _lib.JFA_ERR_INVALID_ARG    # n
    assert f(FAKE, None, 4, 1024, 1e-6, FAKE, FAKE, None) == _lib.JFA_ERR_INVALID_ARG  # n
    assert f(FAKE, None, -1, 128, 1e-6, FAKE, FAKE, None) == _lib.JFA_ERR_INVALID_ARG
    assert f(FAKE, None, 4, 128, -1.0, FAKE, FAKE, None) == _lib.JFA_ERR_INVALID_ARG   # eps
    assert f(FAKE, None, 4, 128, float("nan"), FAKE, FAKE, None) == _lib.JFA_ERR_INVALID_ARG
    assert f(None, None, 4, 128, 1e-6, FAKE, FAKE, None) == _lib.JFA_ERR_INVALID_ARG
    assert f(FAKE + 8, None, 4, 128, 1e-6, FAKE, FAKE, None) == _lib.JFA_ERR_INVALID_ARG
    assert f(FAKE, FAKE + 4, 4, 128, 1e-6, FAKE, FAKE, None) == _lib.JFA_ERR_INVALID_ARG
