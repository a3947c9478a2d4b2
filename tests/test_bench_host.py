"""bench.py's host logic on the CPU: the byte model the roofline divides by,
against the committed traffic figures; the hash guard that voids a traffic
figure once its kernel's sources change; and the refusal of more than one
GPU.  No GPU is involved."""

import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from linear_attention_ssm_chunk_amd import inputs as I  # noqa: E402


def shape_of(index):
    """The sizes bench.algorithmic reads, without drawing the workload's
    values: token count, heads and chunk offsets."""
    w = I.WORKLOADS[index]
    if "nseq" in w:
        lengths, _ = I.ragged_lengths(index, w["nseq"])
    else:
        lengths = [w["T"]] * w["B"]
    cu_chunks = np.concatenate([[0], np.cumsum([-(-L // 64) for L in lengths])])
    return SimpleNamespace(n_tokens=int(sum(lengths)), nk=w["nk"], nv=w["nv"], nseq=len(lengths),
                           cu_chunks=cu_chunks)


def test_shape_of_matches_the_drawn_workload():
    p = I.make_workload(2)
    assert bench.algorithmic(shape_of(2)) == bench.algorithmic(p)


@pytest.mark.parametrize("index", [2, 3, 4, 5])
def test_committed_traffic_matches_the_byte_model(index):
    """Each committed traffic file holds the algorithmic bytes the byte model
    gives now, and HBM bytes counted within 0-5 % above them (no re-reads)."""
    name = I.WORKLOADS[index]["name"]
    by, _ = bench.algorithmic(shape_of(index))
    for stage, kname in bench.KERNELS.items():
        with open(os.path.join(ROOT, "profiles", f"traffic_{kname}_{name}.json")) as f:
            t = json.load(f)
        assert t["algorithmic_bytes_per_launch"] == by[stage], (kname, name)
        assert 1.0 <= t["hbm_bytes_per_launch"] / by[stage] <= 1.05, (kname, name)


def test_decode_traffic_matches_the_byte_model():
    with open(os.path.join(ROOT, "profiles", "traffic_recurrent_decode_decode_B256.json")) as f:
        t = json.load(f)
    sh = bench.DECODE_SHAPE
    assert t["algorithmic_bytes_per_launch"] == bench.decode_bytes(sh["B"], sh["nk"], sh["nv"])


def test_traffic_is_void_once_the_sources_change(monkeypatch):
    name = I.WORKLOADS[3]["name"]
    with open(os.path.join(ROOT, "profiles", f"traffic_{bench.KERNELS[2]}_{name}.json")) as f:
        t = json.load(f)
    monkeypatch.setattr(bench, "source_sha", lambda stage: t["source_sha256"])
    assert bench.traffic_for(2, name) == t["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "source_sha", lambda stage: "0" * 64)
    assert bench.traffic_for(2, name) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2 and "one GPU only" in r.stderr
