"""Collected after the other GPU tests: no bounded in-kernel wait gave up
during any of them (nsa_sel_wait_timeouts; each wait on an LDS counter that
orders a workgroup's waves stops after about 2^18 polls, and a give-up would
mean a launch computed from an incomplete stage).  Runs one NSA workload on
each ring variant first, so the check also means something when the file runs
alone."""
import numpy as np
import pytest

import block_sparse_attention_nsa_amd as nsa
import workloads
from _harness import run_gpu, say

pytestmark = pytest.mark.gpu


def test_no_bounded_wait_gave_up():
    for w in (workloads.make_workload("bf16_T1024"),
              workloads.make_dense(1, 32, 2, 2048, 128, 16, 64, "bf16", "own_first_random", seed=3,
                                   name="g16")):
        out = run_gpu(w)
        assert np.isfinite(out["dq"]).all()
    n = nsa.wait_timeouts()
    say(f"  bounded waits that gave up: {n}")
    assert n == 0
