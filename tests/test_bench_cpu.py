"""bench.py on the host: multi-GPU requests are refused with a message, and counter
summaries are used only for the kernel sources they were taken on."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _bench_module():
    import importlib.util

    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_summary_is_used_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    """roofline.traffic comes from a committed counter summary, and only while the
    kernel's sources hash to the value recorded with it."""
    b = _bench_module()
    (tmp_path / "profiles").mkdir()
    summary = tmp_path / "profiles" / "gemm_fwd_wl_traffic.txt"
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.read_traffic("gemm_fwd", "wl") is None  # no summary
    monkeypatch.setattr(b, "ROOT", ROOT)
    sha = b.kernel_src_sha("gemm_fwd")
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    monkeypatch.setattr(b, "kernel_src_sha", lambda kernel="gemm_fwd": sha)
    summary.write_text(f"# comment\nkernel_src_sha: {sha}\nhbm_bytes_per_launch: 12345\n")
    assert b.read_traffic("gemm_fwd", "wl") == 12345.0
    summary.write_text("kernel_src_sha: 0000000000000000\nhbm_bytes_per_launch: 12345\n")
    assert b.read_traffic("gemm_fwd", "wl") is None  # taken on other sources


def test_source_hash_ignores_comments_and_layout_only():
    """The hash a counter summary is tied to changes with the code and not with
    comments or whitespace; comment markers inside string literals are code."""
    b = _bench_module()
    base = 'int a = 1; // one\nconst char* s = "x // y";\n/* block\n comment */ float f(float x) { return x; }\n'
    same = 'int a = 1;\n// another comment\n  const char* s = "x // y"; float f(float x)\n{ return x; }  /* c */\n'
    assert b.strip_comments(base) == b.strip_comments(same)
    for changed in (base.replace("= 1", "= 2"), base.replace('"x // y"', '"x / y"'),
                    base.replace("return x", "return -x")):
        assert b.strip_comments(changed) != b.strip_comments(base)
