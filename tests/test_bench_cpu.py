"""Host logic of bench.py, on the CPU: the one-GPU guard, the code fingerprint that
decides when a counter summary goes stale, and the copy-calibrated traffic
arithmetic of --summarize-pmc (written into a temporary directory)."""
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_code_only_drops_comments_and_keeps_literals():
    src = ('int a = 1;  // trailing "comment"\n'
           '/* a block\n   comment */ int b = 2;\n'
           '\n'
           'const char *s = "http://x // kept"; char c = \'/\'; char d = \'"\';\n')
    out = bench.code_only(src)
    assert "comment" not in out and "block" not in out
    assert '"http://x // kept"' in out and "'/'" in out and "'\"'" in out
    assert "int a = 1;" in out and "int b = 2;" in out
    assert "\n\n" not in out


def test_kernel_hash_ignores_comments_and_sees_code(tmp_path, monkeypatch):
    csrc = tmp_path / "csrc"
    shutil.copytree(bench.CSRC, csrc)
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    base = bench.kernel_source_hash("gateup_s1")
    hdr = csrc / "dot.h"  # included by the kernel's translation unit
    text = hdr.read_text()
    hdr.write_text(text + "\n// a new comment line\n/* and a block */\n")
    assert bench.kernel_source_hash("gateup_s1") == base
    hdr.write_text(text + "\nconstexpr int kAnotherConstant = 3;\n")
    assert bench.kernel_source_hash("gateup_s1") != base
    hdr.write_text(text)
    unit = csrc / bench.kernel_unit("gateup_s1")
    unit.write_text(unit.read_text().replace("constexpr int", "constexpr  int", 1))
    assert bench.kernel_source_hash("gateup_s1") != base  # spacing inside a line is code text


def write_pmc(path, counter, rows):
    with open(path, "w") as fh:
        fh.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (name, v) in enumerate(rows):
            fh.write(f'{i},"{name}",{counter},{v}\n')


def test_summarize_pmc_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    # the copy kernel moves 1024 MiB each way; FETCH_SIZE reads half of it, WRITE_SIZE all of it
    write_pmc(tmp_path / "cf.csv", "FETCH_SIZE", [("void k_copy(float4 const*, float4*, long)", 524288.0)])
    write_pmc(tmp_path / "cw.csv", "WRITE_SIZE", [("void k_copy(float4 const*, float4*, long)", 1048576.0)])
    kname = "void moe::(anonymous namespace)::k_gateup_s1<3, 0, 1>(moe::FfnArgs)"
    other = "void moe::(anonymous namespace)::k_down_s1<1, 0, true>(moe::FfnArgs)"
    write_pmc(tmp_path / "f.csv", "FETCH_SIZE", [(kname, 100.0), (kname, 120.0), (other, 7.0)])
    write_pmc(tmp_path / "w.csv", "WRITE_SIZE", [(kname, 4.0), (kname, 6.0), (other, 1.0)])
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                        str(tmp_path / "cw.csv"), 1024, ["gateup_s1"])
    out = json.load(open(tmp_path / "profiles" / "traffic_gateup_s1.json"))
    assert out["fetch_scale"] == pytest.approx(2.0) and out["write_scale"] == pytest.approx(1.0)
    assert out["fetch_kib_per_dispatch_raw"] == pytest.approx(110.0)
    assert out["write_kib_per_dispatch_raw"] == pytest.approx(5.0)
    assert out["bytes_per_launch"] == pytest.approx((110.0 * 2 + 5.0) * 1024)
    assert out["source_sha256"] == bench.kernel_source_hash("gateup_s1")
    # a pattern that matches no kernel (or more than one) is refused
    with pytest.raises(SystemExit):
        bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                            str(tmp_path / "cw.csv"), 1024, ["x=gateup_s"])
