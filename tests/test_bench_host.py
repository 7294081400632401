"""Host logic of bench.py that needs no GPU: the source digest that keys committed
hardware-counter summaries to the code they were taken on."""
import json
import os

import bench


def test_code_tokens_drop_comments_keep_literals():
    src = ('int a = 1; // line comment\n/* block\n comment */ const char *s = "http://x /* y */";\n'
           "char q = '/'; char e = '\\''; int b = 2;  /* trailing */\n")
    assert bench.code_tokens(src) == ('int a = 1; const char *s = "http://x /* y */"; '
                                      "char q = '/'; char e = '\\''; int b = 2;")


def test_digest_ignores_comments_and_layout_only():
    a = "__global__ void k(int *p) { p[0] = 1; } // v1\n"
    b = "/* reworded */\n__global__  void k(int *p)\n{\n    p[0] = 1;\n}\n"
    c = "__global__ void k(int *p) { p[0] = 2; }\n"
    assert bench.code_tokens(a) == bench.code_tokens(b)
    assert bench.code_tokens(a) != bench.code_tokens(c)


def test_traffic_only_for_matching_digest(tmp_path, monkeypatch):
    kernel = "gemv_kernel<Q8F32, rows_per_wave=2, waves=8>"
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = {"kernels": {kernel: {"bytes_per_launch": 123, "source_digest": bench.kernel_source_digest(kernel)}}}
    (prof / "traffic.json").write_text(json.dumps(good))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda k="gemv_kernel": good["kernels"][kernel]["source_digest"])
    assert bench.traffic_for(kernel) == 123
    monkeypatch.setattr(bench, "kernel_source_digest", lambda k="gemv_kernel": "0" * 16)
    assert bench.traffic_for(kernel) is None
    assert bench.traffic_for("batch_kernel<16, 2>") is None


def test_every_family_source_exists():
    for fam, files in bench.KERNEL_SOURCES.items():
        for fn in files:
            d = "include" if fn.endswith(".h") else os.path.join("block_quantized_weight_q8_amd", "csrc")
            assert os.path.exists(os.path.join(bench.ROOT, d, fn)), (fam, fn)
        assert len(bench.kernel_source_digest(fam)) == 16


def test_more_than_one_gpu_is_refused():
    """One GPU only: --gpus N > 1 exits with an explanation before touching a device."""
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_help_lists_every_workload():
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--help"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0
    for wl in bench.WORKLOADS:
        assert wl in r.stdout, wl
