"""GPU: a short bench.py run prints one JSON line with every field of the
result contract, consistent with itself."""
import json
import os
import subprocess
import sys

import pytest
import torch

from conftest import ROOT

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def test_bench_line_contract():
    print("[case] bench.py --steps 40 --warmup 4, oracle on the host cores", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "40", "--warmup", "4"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    assert d["unit"] == "tokens/s" and d["n_gpus"] == 1 and d["steps"] == 40 and d["warmup"] == 4
    assert d["higher_is_better"] is True and d["scaling"] == "weak" and d["vs_baseline"] is None
    assert d["dtype"] == "bf16" and d["data"].startswith("synthetic")
    cfg = d["config"]
    assert cfg["workload"] == "llama7b_qkv" and (cfg["n_tokens"], cfg["d"], cfg["d_out"], cfg["k"]) == (32768, 4096, 12288, 64)
    # value is tokens per wall second of the timed steps
    assert d["value"] > 0 and abs(d["value"] * d["ms_per_step"] * 1e-3 - 32768) < 32768 * 1e-3
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["frac"] < 1 and abs(rf["achieved"] / rf["peak"] - rf["frac"]) < 1e-3
    # achieved = algorithmic bytes per launch / average launch time
    assert abs(rf["algorithmic_bytes_per_launch"] / (rf["avg_launch_us"] * 1e-6) / 1e9 - rf["achieved"]) < 0.01 * rf["achieved"]
    assert rf["traffic"] is None or rf["traffic"] >= rf["algorithmic_bytes_per_launch"]
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert cb["cores"] == min(16, os.cpu_count() or 1) and cb["cpu_model"]
    calls = d["calls"]
    assert 0 < calls["kept_fraction"] < 1 and calls["compress_us"] > 0 and calls["wgrad_us"] > 0
    # the generator draw happens inside the timed loop, once per step
    assert calls["host_sampling_us"] > 0
