"""Host logic of the counter summary (jagged_attention_amd.traffic): no GPU needed."""
import csv

from jagged_attention_amd import traffic


def _write(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})


def test_timing_names():
    assert traffic.timing_name("void jfa::(anonymous namespace)::bwd_kv_kernel<128, 4, 0, 1>"
                               "(jfa::BwdParams)") == "jfa_bwd_dkdv"
    assert traffic.timing_name("jfa::(anonymous namespace)::fwd_kernel<128, 4, 0, 1, false>") == \
        "jfa_fwd_bf16"
    assert traffic.timing_name("jfa::(anonymous namespace)::fwd_kernel<128, 4, 0, 1, true>") == \
        "jfa_fwd_mxfp8"
    assert traffic.timing_name("void jfa::(anonymous namespace)::bwd_kvq_kernel<128, 4, 0, 1>"
                               "(jfa::BwdParams)") == "jfa_bwd_kvq"
    assert traffic.timing_name("jfa::(anonymous namespace)::fwd_kernel<128, 4, 0, 1, true, false>"
                               ) == "jfa_fwd_mxfp8"
    assert traffic.timing_name("jfa::(anonymous namespace)::bwd_kvq_kernel<128, 4, 0, 0, false, "
                               "true>(jfa::BwdParams)") == "jfa_bwd_kvq_mxfp8"
    assert traffic.timing_name("jfa::(anonymous namespace)::bwd_q1_kernel<128, 1, 0, false>"
                               "(jfa::BwdParams)") == "jfa_bwd_dq"
    assert traffic.timing_name("jfa::(anonymous namespace)::bwd_q_db_kernel<64, 2, 2, 2, false>"
                               ) == "jfa_dbias_dq"
    assert traffic.timing_name("__amd_rocclr_copyBuffer") == "copy"
    assert traffic.timing_name("something_else") is None


def test_summary_scales_by_the_copy(tmp_path):
    mib = 64
    # the counters read half the true bytes for the copy: every kernel is scaled by 2
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    _write(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", mib * 1024 / 2),
                                 ("bwd_kv_kernel<128, 4, 0, 1>", 1000.0),
                                 ("bwd_kv_kernel<128, 4, 0, 1>", 3000.0)])
    _write(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", mib * 1024 / 4),
                                 ("bwd_kv_kernel<128, 4, 0, 1>", 100.0),
                                 ("bwd_kv_kernel<128, 4, 0, 1>", 100.0)])
    kernels, calib = traffic.summarize(str(fetch), str(write), mib << 20)
    e = kernels["jfa_bwd_dkdv"]
    assert e["fetch_bytes"] == 2000 * 1024 * 2
    assert e["write_bytes"] == 100 * 1024 * 4
    assert e["bytes_per_launch"] == e["fetch_bytes"] + e["write_bytes"]
    assert calib["fetch_factor"] == 2.0 and calib["write_factor"] == 4.0


def test_per_kernel_source_hash():
    # a kernel's counters stay valid across edits to other kernels' files
    a = traffic.source_hash("jfa_bwd_dkdv")
    assert a == traffic.source_hash("jfa_bwd_dq")          # same source file
    assert a != traffic.source_hash("jfa_fwd_bf16")
    assert traffic.source_hash() not in (a, traffic.source_hash("jfa_fwd_bf16"))
