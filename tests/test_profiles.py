"""The committed HBM byte counters (`profiles/hbm_traffic.json`: rocprofv3
FETCH_SIZE and WRITE_SIZE per dispatch, scaled by what the same counters read
for a plain device copy) against the algorithmic bytes of each workload.

- They were taken on the current kernel sources (the hash `bench.py` checks
  before it reports `roofline.traffic`).
- An unsplit forward moves no expanded (B, L, D, N) state through HBM: such a
  tensor in fp32 would add 4N = 64 bytes per (b, t, d), several times the
  workload's algorithmic bytes, where the counters stay within 10% of them
  (reading guide of arXiv 2312.00752, "Donanım Duyarlı Durum Genişletme": the
  expanded state lives only in on-chip memory).
- A split forward's excess is its first pass, which reads u, delta and B once
  more for every segment but the last.
"""
from __future__ import annotations

import json
import os

import pytest
import torch

import bench
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
    TRAFFIC = json.load(f)


def _kind(name):
    return "decode" if name.startswith("decode") else "bwd" if "-bwd" in name else "fwd"


@pytest.mark.parametrize("name", sorted(TRAFFIC))
def test_counters_were_taken_on_the_current_sources(name):
    assert TRAFFIC[name]["source_sha"] == bench._source_sha(*bench.SHA_FILES[_kind(name)]), (
        f"{name}: kernel sources changed since its HBM counters were taken")


@pytest.mark.parametrize("name", ["mamba-370m-layer-fwd", "mamba-2.8b-layer-fwd",
                                  "mamba-2.8b-layer-fwd-conv4", "decode-state-update"])
def test_no_expanded_state_in_hbm(name):
    t = TRAFFIC[name]
    assert t["algorithmic_bytes"] <= t["bytes_per_step"] <= 1.10 * t["algorithmic_bytes"]


@pytest.mark.parametrize("name,idx", [("million-length-fwd", 4), ("mamba-2.8b-32k-fwd", 5)])
def test_split_forward_excess_is_the_first_pass(name, idx):
    import selective_state_space_10_amd as ssm
    w = WORKLOADS[idx]
    plan = ssm.scan_fwd_plan(w.batch, w.seqlen, w.dim, w.dstate, w.io_dtype)
    S = plan["segments"]
    assert S > 1
    io = 4 if w.io_dtype == torch.float32 else 2
    first_pass = (S - 1) / S * (2 * w.batch * w.seqlen * w.dim + w.batch * w.seqlen * w.dstate) * io
    t = TRAFFIC[name]
    assert t["algorithmic_bytes"] + 0.9 * first_pass <= t["bytes_per_step"]
    assert t["bytes_per_step"] <= 1.10 * (t["algorithmic_bytes"] + first_pass)
