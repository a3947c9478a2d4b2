"""bench.py's host logic on the CPU: the irreducible byte model the roofline
divides by, pinned to the workload arithmetic worked out by hand; the
implementation's byte model against the committed traffic figures; the hash
guard that voids a traffic figure once its kernel's sources change; and the
refusal of more than one GPU.  No GPU is involved."""

import json
import os
import subprocess
import sys
import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from linear_attention_ssm_chunk_amd import inputs as I  # noqa: E402


def shape_of(index):
    """The sizes bench.algorithmic reads, without drawing the workload's
    values (bench.workload_shape)."""
    return bench.workload_shape(index)


def test_shape_of_matches_the_drawn_workload():
    p = I.make_workload(2)
    assert bench.algorithmic(shape_of(2)) == bench.algorithmic(p)


def test_irreducible_bytes_of_the_batched_workload():
    """B=4, T=8192, nk=16, nv=32 with entry states, worked by hand: q and k
    2 x 32768 x 16 x 128 x 2 B, v and o 32768 x 32 x 128 x 2 B each, g and
    beta 32768 x 32 x 8 B, the state 2 x 4 x 32 x 64 KiB, the entry states
    512 chunks x 32 heads x 32 KiB: 0.83 GB plus 0.54 GB."""
    per, total = bench.irreducible(shape_of(3), entry=True)
    qk, v, o, gb = 268435456, 268435456, 268435456, 8388608
    state, s_out = 16777216, 536870912
    assert per == {1: gb, 2: qk + v + o + s_out + state}
    assert total == 1367343104
    assert round((qk + v + o + gb + state) / 1e9, 2) == 0.83 and round(s_out / 1e9, 2) == 0.54
    per0, total0 = bench.irreducible(shape_of(3), entry=False)
    assert total0 == total - s_out


def test_each_workload_asks_for_entry_states_only_where_stated():
    assert bench.workload_flags(I.WORKLOADS[3]) == bench.OPT_ENTRY_STATES
    for index in (1, 2, 4, 5):
        assert bench.workload_flags(I.WORKLOADS[index]) == 0
    assert bench.workload_flags(I.WORKLOADS[5], raw_qk=True) == bench.OPT_L2NORM_QK


@pytest.mark.parametrize("index", [2, 3, 4, 5])
def test_committed_traffic_matches_the_byte_model(index):
    """Each committed traffic file taken on the current kernel sources holds
    the bytes the implementation's byte model gives now for the workload's
    options, and HBM bytes counted within 0-5 % above them (no re-reads)."""
    name = I.WORKLOADS[index]["name"]
    by, _ = bench.algorithmic(shape_of(index), bench.workload_flags(I.WORKLOADS[index]))
    for stage, kname in bench.KERNELS.items():
        path = os.path.join(ROOT, "profiles", f"traffic_{kname}_{name}.json")
        if not os.path.exists(path):
            pytest.skip(f"{path} not taken on the current kernels")
        with open(path) as f:
            t = json.load(f)
        assert t["source_sha256"] == bench.source_sha(stage), f"{path} is stale"
        assert t["algorithmic_bytes_per_launch"] == by[stage], (kname, name)
        assert 1.0 <= t["hbm_bytes_per_launch"] / by[stage] <= 1.05, (kname, name)


def test_decode_traffic_matches_the_byte_model():
    path = os.path.join(ROOT, "profiles", "traffic_recurrent_decode_decode_B256.json")
    if not os.path.exists(path):
        pytest.skip(f"{path} not taken on the current kernels")
    with open(path) as f:
        t = json.load(f)
    assert t["source_sha256"] == bench.source_sha(3), f"{path} is stale"
    sh = bench.DECODE_SHAPE
    assert t["algorithmic_bytes_per_launch"] == bench.decode_bytes(sh["B"], sh["nk"], sh["nv"])


def test_traffic_is_void_once_the_sources_change(monkeypatch, tmp_path):
    name = I.WORKLOADS[3]["name"]
    t = {"source_sha256": "a" * 64, "hbm_bytes_per_launch": 12345}
    (tmp_path / "profiles").mkdir()
    with open(tmp_path / "profiles" / f"traffic_{bench.KERNELS[2]}_{name}.json", "w") as f:
        json.dump(t, f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_sha", lambda stage: t["source_sha256"])
    assert bench.traffic_for(2, name) == t["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "source_sha", lambda stage: "0" * 64)
    assert bench.traffic_for(2, name) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2 and "one GPU only" in r.stderr
