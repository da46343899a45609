"""Host-side checks of bench.py: the refusal of several GPUs, the roofline record,
and the table of counter summaries it reads (every entry names a committed
summary of its own kernel source with a per-launch byte count, taken on the code
that source holds now)."""
import os
import re
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_roofline_record_and_traffic_above_peak():
    r = bench.roofline(8e9, 2e-3, traffic=8.8e9)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.HBM_PEAK_GBS
    assert abs(r["achieved"] - 4000.0) < 1e-6 and abs(r["frac"] - 0.5) < 1e-9
    assert r["traffic"] == 8.8e9 and abs(r["traffic_GBps"] - 4400.0) < 1e-6
    over = bench.roofline(8e9, 1e-3, traffic=9e9)  # 9 TB/s counted: above the peak
    assert over["traffic"] is None and "traffic_note" in over
    assert bench.roofline(1e9, 1e-3)["traffic"] is None


def test_every_profile_entry_names_its_summary():
    for key, (src, fname) in bench.PROFILE_OF.items():
        assert key in bench.OPS, key
        assert os.path.exists(os.path.join(ROOT, "gated_delta_rule_short_amd", "csrc", src)), src
        text = open(os.path.join(ROOT, "profiles", fname)).read()
        assert re.search(r"kernel_source:\s*%s\b" % re.escape(src), text), fname
        assert re.search(r"kernel_source_sha:\s*[0-9a-f]{16}", text), fname
        assert re.search(r"hbm_bytes_per_launch:\s*[0-9.eE+]+", text), fname
        assert "--only %s " % key in text, fname  # the command that made it times this entry


def test_every_profile_summary_describes_the_current_code():
    # a kernel edited after its summaries were taken leaves the bench line without
    # counted traffic and busy fractions: take the summaries again (rocprofv3, the
    # commands each summary names) when this fails
    for key, (src, fname) in bench.PROFILE_OF.items():
        assert bench._profile_field(key, "hbm_bytes_per_launch") is not None, (key, fname, src)


def test_source_hash_ignores_comments_and_layout(tmp_path, monkeypatch):
    csrc = tmp_path / "gated_delta_rule_short_amd" / "csrc"
    csrc.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    f = csrc / "k.hip"
    f.write_text("// header\nint f(int a) {\n    return a + 1;  /* one */\n}\n")
    h = bench._source_sha("k.hip")
    f.write_text("// another header\n/* block\n comment */ int f(int a) { return a + 1; }\n")
    assert bench._source_sha("k.hip") == h
    f.write_text("int f(int a) { return a + 2; }\n")
    assert bench._source_sha("k.hip") != h
