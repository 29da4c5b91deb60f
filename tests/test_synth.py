"""The seeded input generator: shapes, reproducibility, attention concentration."""

import math

import numpy as np
import torch

from synth import f90_fraction, make_video_qkv, workload, WORKLOADS


def test_shapes_dtypes_and_seed_reproducibility():
    a = make_video_qkv(2, 8, 8, 2, 32, "bf16", seed=5)
    b = make_video_qkv(2, 8, 8, 2, 32, "bf16", seed=5)
    c = make_video_qkv(2, 8, 8, 2, 32, "bf16", seed=6)
    assert a["q"].shape == (1, 2, 128, 32) and a["q"].dtype == torch.bfloat16
    assert torch.equal(a["k"], b["k"]) and torch.equal(a["q"], b["q"])
    assert not torch.equal(a["k"], c["k"])


def test_concentration_is_calibrated_per_head():
    targets = [0.04, 0.10]
    x = make_video_qkv(4, 16, 16, 2, 64, "fp32", seed=1, f90_targets=targets)
    for h, t in enumerate(targets):
        q = x["q"][0, h].double()
        k = x["k"][0, h].double()
        logits = (q[x["calib_idx"]] @ k.T) / math.sqrt(64)
        srt, _ = torch.sort(logits, dim=1, descending=True)
        assert abs(float(f90_fraction(srt, 1.0).mean()) - t) < 0.005


def test_workload_table_matches_the_call_shapes():
    assert WORKLOADS["c1_tiny_fp32"].n == 1024 and WORKLOADS["c1_tiny_fp32"].dtype == "fp32"
    assert WORKLOADS["c2_dit_8k"].n == 8192
    assert WORKLOADS["c3_dit_32k"].n == 32760 and WORKLOADS["c3_dit_32k"].heads == 40
    assert WORKLOADS["c4_long_75k"].n == 75600
    t = workload("c3_dit_32k").f90_targets()
    assert np.isclose(t[0], 0.03) and np.isclose(t[-1], 0.12)
