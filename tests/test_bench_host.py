"""Host logic of bench.py (CPU only): the code digest that ties a committed counter summary to the
kernel source it was taken on, and the lookup of the stored traffic figure."""
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_only_drops_comments_and_layout():
    a = "int f(int x) {\n  // note\n  return x + 1; /* more */\n}\n"
    b = "int f(int x) { return x + 1;\n}   // other note\n"
    assert bench._code_only(a) == bench._code_only(b)


def test_code_only_keeps_literals_and_code_changes():
    assert '"//not a comment"' in bench._code_only('const char* s = "//not a comment"; // real')
    assert "'/'" in bench._code_only("char c = '/'; /* x */")
    assert bench._code_only('s = "a\\"//b";') == 's = "a\\"//b";'
    assert bench._code_only("return x + 1;") != bench._code_only("return x + 2;")


def test_stored_traffic_only_for_current_code(tmp_path, monkeypatch):
    csrc = tmp_path / "sparse_mixture_experts_33_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (csrc / "k.hip").write_text("__global__ void k() {}  // v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    digest = bench.source_digest(["k.hip"])
    (tmp_path / "profiles" / "traffic_k_w.md").write_text(
        f"source_files: k.hip\nsource_digest: {digest}\nhbm_bytes_per_launch: 1.5e9\n")
    assert bench.stored_traffic("k", "w") == 1.5e9
    (csrc / "k.hip").write_text("// a comment only\n__global__ void k() {}\n")
    assert bench.stored_traffic("k", "w") == 1.5e9
    (csrc / "k.hip").write_text("__global__ void k() { int a = 0; }\n")
    assert bench.stored_traffic("k", "w") is None
    assert bench.stored_traffic("k", "other") is None


def test_committed_summaries_name_existing_sources():
    pdir = os.path.join(ROOT, "profiles")
    csrc = os.path.join(ROOT, "sparse_mixture_experts_33_amd", "csrc")
    for name in os.listdir(pdir):
        txt = open(os.path.join(pdir, name)).read()
        f = re.search(r"source_files:\s*([^\n]+)", txt)
        if f:
            for src in f.group(1).split():
                assert os.path.exists(os.path.join(csrc, src)), (name, src)
            assert re.search(r"source_digest:\s*[0-9a-f]{16}\b", txt), name


def _smi_block(watts, mhz):
    gfx = "".join(f"        GFX_{i}:\n            CLK: {mhz + i} MHz\n            MIN_CLK: 500 MHz\n"
                  f"            MAX_CLK: 2400 MHz\n" for i in range(8))
    return (f"GPU: 0\n    POWER:\n        SOCKET_POWER: {watts} W\n        GFX_VOLTAGE: N/A\n    CLOCK:\n{gfx}"
            "        MEM_0:\n            CLK: 2000 MHz\n            MIN_CLK: 2000 MHz\n")


def test_parse_power_keeps_samples_inside_the_timed_steps():
    text = ("GPU[0]\t\t: Max Graphics Package Power (W): 1400.0\n"
            + "T 100.0\n" + _smi_block(250, 150)      # in the first second of the timed steps: dropped
            + "T 101.0\n" + _smi_block(1390, 2190)
            + "T 102.0\n" + _smi_block(1400, 2200)
            + "T 103.0\n" + _smi_block(1398, 2210)
            + "T 104.9\n" + _smi_block(300, 160))     # during the last half second: dropped
    p = bench.parse_power(text, 100.0, 105.0)
    assert p["samples"] == 3 and p["power_cap_w"] == 1400.0
    assert p["socket_w_median"] == 1398 and p["socket_w_min"] == 1390 and p["socket_w_max"] == 1400
    # the clock of a sample is the mean over the eight GFX domains (MEM_0's clock is not one of them)
    assert p["gfx_mhz_median"] == 2203.5 and p["gfx_mhz_min"] == 2193.5


def test_parse_power_without_samples():
    p = bench.parse_power("", 0.0, 10.0)
    assert p["samples"] == 0 and p["socket_w_median"] is None and p["power_cap_w"] is None
