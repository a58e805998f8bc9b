"""CPU tests of bench.py's host logic: the source hash that decides whether stored
rocprofv3 traffic counters still describe the current kernel."""
import json
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _tree(tmp_path, files):
    for rel, text in files.items():
        p = tmp_path / rel
        p.parent.mkdir(parents=True, exist_ok=True)
        p.write_text(text)
    return str(tmp_path)


def test_kernel_hash_follows_local_includes(tmp_path):
    root = _tree(tmp_path, {
        "bit_diffusion_model_svdq_amd/csrc/k.hip": '#include "tail.h"\n#include <vector>\nint k;\n',
        "bit_diffusion_model_svdq_amd/csrc/tail.h": '#include "api.h"\nint t;\n',
        "include/api.h": "int a;\n",
        "bit_diffusion_model_svdq_amd/csrc/other.h": "int o;\n",
    })
    h0 = bench.kernel_source_hash("k.hip", root)
    assert h0 == bench.kernel_source_hash("k.hip", root)
    # a header two levels down, in include/, changes the hash
    (tmp_path / "include/api.h").write_text("int a2;\n")
    h1 = bench.kernel_source_hash("k.hip", root)
    assert h1 != h0
    # a header the kernel does not include leaves it alone
    (tmp_path / "bit_diffusion_model_svdq_amd/csrc/other.h").write_text("int o2;\n")
    assert bench.kernel_source_hash("k.hip", root) == h1
    # the kernel file itself
    (tmp_path / "bit_diffusion_model_svdq_amd/csrc/k.hip").write_text('#include "tail.h"\nint k2;\n')
    assert bench.kernel_source_hash("k.hip", root) != h1


def test_kernel_hash_missing_header_raises(tmp_path):
    root = _tree(tmp_path, {"bit_diffusion_model_svdq_amd/csrc/k.hip": '#include "gone.h"\n'})
    with pytest.raises(FileNotFoundError):
        bench.kernel_source_hash("k.hip", root)


@pytest.mark.parametrize("kernel", ["k1_smooth_quant.hip", "k2_w4a4_gemm.hip", "k2_mxfp4_gemm.hip"])
def test_kernel_hash_resolves_every_header_of_the_library(kernel):
    assert len(bench.kernel_source_hash(kernel)) == 16


def test_stored_traffic_is_dropped_when_the_source_changes(tmp_path, monkeypatch):
    stored = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    workload, entries = next((w, e) for w, e in stored.items() if w != "calibration")
    kernel, entry = next(iter(entries.items()))
    fake = tmp_path / "profiles"
    fake.mkdir()
    entry = dict(entry, source_sha256_16=bench.kernel_source_hash(kernel))
    (fake / "traffic.json").write_text(json.dumps({workload: {kernel: entry}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda name: entry["source_sha256_16"])
    assert bench.load_traffic(kernel, workload) == entry["bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda name: "0" * 16)
    assert bench.load_traffic(kernel, workload) is None


def test_host_cpu_record():
    """cpu_baseline's host fields: the CPUs this process may use and the CPU model."""
    h = bench.host_cpu()
    assert isinstance(h["nproc"], int) and h["nproc"] >= 1
    assert h["cpu_model"] is None or isinstance(h["cpu_model"], str)
    assert bench.blas_threads() >= 1


def test_sclk_reader_tolerates_missing_sysfs():
    """The engine-clock reading is an int (MHz) or None, never an exception."""
    v = bench.read_sclk_mhz()
    assert v is None or (isinstance(v, int) and v > 0)
