"""bench.py's host logic, without a GPU: the one-GPU contract, the FLOP and
byte counts it divides by, and the rule that counter figures from a
committed profile are used only while the kernel source they were taken on
is unchanged."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       capture_output=True, text=True, timeout=120,
                       env={**os.environ, **env})
    assert r.returncode == 2
    assert "GPU" in r.stderr and r.stdout == ""


def test_flop_and_byte_counts():
    # QK^T + PV of the full-context layer: 4 * 8 * 8192^2 * 128
    assert bench.attn_flops(1, 8192) == 4 * 8 * 8192 ** 2 * 128 == 274877906944
    # value width 192: 2 * 8 * S^2 * (128 + 192)
    assert bench.attn_flops(1, 8192, Dv=192) == 2 * 8 * 8192 ** 2 * 320
    # one GPU's share: 1024 queries against 8192 keys
    assert bench.attn_flops(1, 8192, Sq=1024) == 4 * 8 * 1024 * 8192 * 128
    # projection: pair bf16 read, weight read, fp32 bias written
    assert bench.proj_bytes(512, 128) == 512 * 512 * 128 * 2 + 128 * 8 * 2 + 8 * 512 * 512 * 4
    assert bench.proj_flops(512, 128) == 2 * 512 * 512 * 128 * 8


def _copy_tree(tmp_path):
    root = tmp_path / "repo"
    (root / "long_context_biased_amd" / "csrc").mkdir(parents=True)
    (root / "profiles").mkdir()
    for f in ("biased_mqa_fwd.hip", "abg_internal.h"):
        shutil.copy(os.path.join(ROOT, "long_context_biased_amd", "csrc", f),
                    root / "long_context_biased_amd" / "csrc" / f)
    shutil.copy(bench.COUNTERS_FILE, root / "profiles" / os.path.basename(bench.COUNTERS_FILE))
    return root


def test_counters_follow_the_kernel_code(tmp_path, monkeypatch):
    root = _copy_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    monkeypatch.setattr(bench, "COUNTERS_FILE",
                        str(root / "profiles" / os.path.basename(bench.COUNTERS_FILE)))
    digest = bench.source_digest()
    counters = bench.load_counters("pair")
    assert counters is not None, "the committed counters do not match the committed kernel"
    assert counters["mfma_flops_per_launch"] == bench.attn_flops(1, 8192)
    assert bench.load_counters("two") is None  # taken on the other route
    src = root / "long_context_biased_amd" / "csrc" / "biased_mqa_fwd.hip"
    text = src.read_text()
    # comments and white space do not count
    src.write_text(text.replace("\n", "\n  // a new comment line\n", 3))
    assert bench.source_digest() == digest
    assert bench.load_counters("pair") is not None
    # code does
    src.write_text(text.replace("constexpr int kTileKeys = 64;", "constexpr int kTileKeys = 64 ;\nint x_;", 1))
    assert bench.source_digest() != digest
    assert bench.load_counters("pair") is None
