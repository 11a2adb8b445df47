"""Host-side logic of bench.py, without a GPU: the one-GPU guard, the kernel
names it attributes timings and counters to (they must be the template
instances the library launches, as recorded by the profiler in the committed
summaries), the counted-traffic lookup and the roofline arithmetic."""

import glob
import hashlib
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import get_config  # noqa: E402


def _profile_text():
    return "\n".join(open(p).read() for p in sorted(glob.glob(os.path.join(ROOT, "profiles",
                                                                           "*.md"))))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("name", ["batched_mix", "mistral7b", "qwen25_7b_2tier", "gemma2_9b"])
def test_kernel_names_are_the_profiled_instances(name):
    """The score and pack/unpack kernels bench.py names for a workload appear
    in the kernel traces the profiler recorded for it."""
    cfg = get_config(name)
    text = _profile_text()
    names = bench.score_kernel_names(cfg.q_heads, cfg.kv_heads, cfg.head_dim)
    nb = bench.pack_batch(cfg.kv_heads, cfg.head_dim)
    names["pack"] = f"pack_kernel<{cfg.head_dim},{nb}>"
    names["unpack"] = f"unpack_kernel<{cfg.head_dim},{nb},true>"
    for stage, k in names.items():
        assert f"`{k}`" in text, (name, stage, k)


def test_pack_batch_rule():
    # 2*Hkv rows at 64/(d/8) rows a step, rounded up to a power of two, at most 8
    assert bench.pack_batch(8, 128) == 4
    assert bench.pack_batch(8, 256) == 8
    assert bench.pack_batch(4, 128) == 2
    assert bench.pack_batch(2, 64) == 1
    assert bench.pack_batch(16, 256) == 8


def test_counted_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    """A summary's traffic figure is used only while the kernel's source file
    still has the hash recorded beside it."""
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel source v1")
    good = hashlib.sha256(b"kernel source v1").hexdigest()
    stale = hashlib.sha256(b"kernel source v0").hexdigest()
    (tmp_path / "profiles" / "p.md").write_text(
        f"<!-- traffic workload=w kernel=a<1> bytes_per_launch=123 source=k.hip sha256={good} -->\n"
        f"<!-- traffic workload=w kernel=b<1> bytes_per_launch=456 source=k.hip sha256={stale} -->\n"
        f"<!-- traffic workload=v kernel=a<1> bytes_per_launch=789 source=gone.hip sha256={good} -->\n")
    monkeypatch.setattr(bench, "__file__", str(tmp_path / "bench.py"))
    assert bench.counted_traffic("a<1>", "w") == 123
    assert bench.counted_traffic("b<1>", "w") is None        # source changed since
    assert bench.counted_traffic("a<1>", "v") is None        # source missing
    assert bench.counted_traffic("a<1>", "u") is None        # no summary for the workload
    src.write_bytes(b"kernel source v2")
    assert bench.counted_traffic("a<1>", "w") is None


def test_committed_traffic_tags_of_the_score_passes_are_current():
    """The score kernels' counter summaries were taken on today's score.hip."""
    for wl in ("batched_mix", "mistral7b", "qwen25_7b_2tier", "gemma2_9b"):
        cfg = get_config(wl)
        for k in bench.score_kernel_names(cfg.q_heads, cfg.kv_heads, cfg.head_dim).values():
            assert bench.counted_traffic(k, wl) is not None, (wl, k)


def test_every_profiled_source_hash_is_current():
    """Every profile summary names the sha256 of the kernel source it was
    taken on (traffic tags, and the counter summaries' source lines) and of
    the build script whose flags compiled it; each must be the file as it is
    now, so a summary cannot outlive the code it describes."""
    import re
    seen = 0
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        text = open(path).read()
        refs = re.findall(r"source=(\S+) sha256=([0-9a-f]{64})", text)
        refs += re.findall(r"`?(serving_sk_score_amd/(?:csrc/\w+\.(?:hip|cpp)|build\.py))`? "
                           r"sha256 `?([0-9a-f]{64})", text)
        for src, sha in refs:
            cur = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
            assert cur == sha, (os.path.basename(path), src)
            seen += 1
    assert seen > 0


def test_roofline_arithmetic():
    r = bench.hbm_rl(8e9, 2e-3, "no_such_kernel<1>", "batched_mix", launches=2)
    assert r["achieved"] == 4000.0 and r["frac"] == 0.5
    assert r["bytes_per_launch"] == 4_000_000_000 and r["avg_launch_ms"] == 1.0
    assert r["traffic"] is None
    m = bench.mfma_rl(np.array([1e12, 3e12]), np.array([1.0, 1.0]), "no_such_kernel<1>",
                      "batched_mix")
    assert m["achieved"] == 2000.0 and m["frac"] == 0.8
    assert m["flops_per_launch"] == 2e12 and m["avg_launch_ms"] == 1.0


def test_step_spread_sums_a_stage_per_step():
    """Per-stage median and minimum over steps, a stage summing its labels'
    launches within each step."""
    res = [{"a": (np.array([1.0, 2.0]), None), "b": (np.array([4.0]), None)},
           {"a": (np.array([0.5]), None), "b": (np.array([1.0, 1.0]), None)},
           {"a": (np.array([3.0]), None), "b": (np.array([0.0]), None)}]
    out = bench.step_spread(res, {"a": ["a"], "ab": ["a", "b"]})
    assert out["a"] == [3.0, 0.5]          # per step 3.0, 0.5, 3.0
    assert out["ab"] == [3.0, 2.5]         # per step 7.0, 2.5, 3.0
