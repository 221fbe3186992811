"""Host logic of bench.py (no GPU): the one-GPU guard, the metric's flop
count, and the rule that ties roofline.traffic to the kernel sources the
counters were taken on."""

import importlib.util
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = ("transformer_exact_attention_flashattention_amd/csrc/fa_kernels.h",
           "transformer_exact_attention_flashattention_amd/csrc/fa_fwd.hip")


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a run that did not happen


def test_sweep_dtype_is_checked_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--sweep", "--sweep-dtype", "f32"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "--sweep-dtype" in r.stderr
    assert r.stdout == ""


def test_metric_flops(bench):
    c = {"B": 1, "H": 16, "N": 16384, "D": 256, "causal": True}
    assert bench.metric_flops(c) == 4.0 * 16 * 16384 ** 2 * 256 / 2
    c["causal"] = False
    assert bench.metric_flops(c) == 4.0 * 16 * 16384 ** 2 * 256


def copy_sources(dst):
    for rel in SOURCES:
        os.makedirs(os.path.join(dst, os.path.dirname(rel)), exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), os.path.join(dst, rel))


def test_digest_ignores_comments_but_not_code(bench, tmp_path, monkeypatch):
    copy_sources(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.kernel_source_digest()
    hip = tmp_path / SOURCES[1]
    text = hip.read_text()
    hip.write_text("// a new comment line\n\n" + text.replace("\n", "  /* trailing */\n", 1))
    assert bench.kernel_source_digest() == d0
    hip.write_text(text.replace("constexpr int kMaxSplits = 64;", "constexpr int kMaxSplits = 63;"))
    assert bench.kernel_source_digest() != d0


def test_traffic_only_for_matching_sources(bench, tmp_path, monkeypatch):
    good = {"kernel_sha256": bench.kernel_source_digest(), "hbm_bytes_per_launch": 1.25e9}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(good))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.load_traffic(0) == 1.25e9
    f.write_text(json.dumps(dict(good, kernel_sha256="0" * 64)))
    assert bench.load_traffic(0) is None
    f.write_text("not json")
    assert bench.load_traffic(0) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.load_traffic(0) is None


def test_committed_traffic_file_is_well_formed(bench):
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert len(t["kernel_sha256"]) == 64
    assert t["hbm_bytes_per_launch"] > 0


def test_hwmon_power_dir(bench, tmp_path, monkeypatch):
    hw = tmp_path / "card0" / "device" / "hwmon" / "hwmon3"
    hw.mkdir(parents=True)
    (tmp_path / "card1" / "device" / "hwmon" / "hwmon0").mkdir(parents=True)  # no power reading
    pattern = str(tmp_path / "card*" / "device" / "hwmon" / "hwmon*")
    real_glob = bench.glob.glob
    monkeypatch.setattr(bench.glob, "glob", lambda p: real_glob(pattern))
    assert bench.hwmon_power_dir() is None
    (hw / "power1_input").write_text("1387000000\n")
    assert bench.hwmon_power_dir() == str(hw)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_model_check_verdict(bench, dtype):
    """The bench's rounding-model comparison: the model's own output passes
    with ratio 0; one element moved by 0.25 (beyond 2 ulp + 2 u' max P max|V|
    for any |O| < 4 and |V| < 5) fails the per-element bound; a systematic
    one-unit shift of every element stays within the bound but fails the
    share of differing elements."""
    import torch

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from kernel_model import forward_model, output_ulp
    from transformer_exact_attention_flashattention_amd import inputs

    q, k, v = inputs.make_qkv(1, 2, 200, 64, dtype, seed=11)
    om, _ = forward_model(q, k, v, 0.125, True)
    r = bench.model_check(om, q, k, v, 0.125, True)
    assert r["model_ok"] and r["worst_ratio_to_model_bound"] == 0.0 and r["frac_differing"] == 0.0
    bad = om.clone()
    assert float(v.abs().max()) < 5.0 and float(om.abs().max()) < 4.0
    bad[0, 1, 100, 7] += 0.25
    r = bench.model_check(bad, q, k, v, 0.125, True)
    assert not r["model_ok"] and r["worst_ratio_to_model_bound"] > 1.0
    ulp = torch.from_numpy(output_ulp(om.double().numpy(), q.dtype))
    shifted = (om.double() + ulp).to(q.dtype)
    r = bench.model_check(shifted, q, k, v, 0.125, True)
    assert r["worst_ratio_to_model_bound"] <= 1.0 and r["frac_differing"] > 0.5 and not r["model_ok"]
