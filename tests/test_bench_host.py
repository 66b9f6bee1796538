"""Host logic of bench.py (CPU only): kernel names from the profiler's
trace, and the stored HBM traffic that is reported only while the kernel
sources are the ones it was measured on."""
import json

import bench


def test_kernel_names():
    assert bench._short("void gdn::(anonymous namespace)::chain_bf16_kernel<128, false, 8, 2, true>"
                        "(gdn::ChainLaunch)") == "chain_bf16_kernel<128, false, 8, 2, true>"
    assert bench._short("_ZN3gdn12_GLOBAL__N_113decode_kernelILi128EDF16bEEvNS_12DecodeLaunchE") == \
        "decode_kernel<128, bf16>"
    assert bench._short("_ZN3gdn12_GLOBAL__N_116scalar_op_kernelILi64ELi128EfEEvNS_14ScalarOpLaunchE") == \
        "scalar_op_kernel<64, 128, float>"


def test_measured_traffic_follows_the_sources(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    rec = dict(workload="w", sources_sha256="x", hbm_bytes_per_call=300,
               kernels={"a_kernel<1>": dict(fetch_bytes=100.4, write_bytes=50.0),
                        "b_kernel": dict(fetch_bytes=150.0, write_bytes=0.0)})
    (tmp_path / "profiles" / "traffic_w.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "sources_sha256", lambda: "x")
    assert bench.measured_traffic("w") == 300
    assert bench.measured_traffic("w", "a_kernel") == 150
    assert bench.measured_traffic("w", "c_kernel") is None
    assert bench.measured_traffic("other") is None
    monkeypatch.setattr(bench, "sources_sha256", lambda: "y")
    assert bench.measured_traffic("w") is None


def test_source_hash_ignores_comments_and_whitespace():
    # the counter summaries stay valid across comment edits, not across code edits
    import bench
    a = 'int f(int x) { // twice\n  return 2 * x; /* doubled */ }\nconst char *s = "a // b";\n'
    b = 'int  f(int x)\n{\n  return 2*x;\n}\nconst char *s = "a // b";  // the same code\n'
    c = 'int f(int x) { return 3 * x; }\nconst char *s = "a // b";\n'
    d = 'int f(int x) { return 2 * x; }\nconst char *s = "a /* b";\n'
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
    assert bench.code_text(a) != bench.code_text(d)    # string contents are code
