"""CPU: the algorithmic work the roofline figures divide by, and the one-GPU guard of bench.py.

The bytes a step must move are W once (V x H elements), the block's hidden rows once and the
per-row state; the flops are 2 M V H (the [M][V] logits are never stored).  The figures below
are written out from the workload shapes by hand, independently of bench.py's helper.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    sys.path.insert(0, ROOT)
    import bench as b
    return b


def test_batch_one_threshold_work(bench):
    from decoding_step_amd.workloads import WORKLOADS
    nbytes, flops = bench.algorithmic_work(WORKLOADS["threshold_b1_l32"])
    w = 126464 * 2048 * 2                   # bf16 W
    h = 32 * 2048 * 2                       # bf16 hidden rows of the block
    state = 32 * (1 + 1 + 4 + 1 + 4 + 4)    # mask in and out, token, commit, confidence, gap
    assert nbytes == w + h + state == 518_128_096
    assert flops == 2 * 32 * 126464 * 2048 == 16_575_889_408


def test_batched_mixed_work(bench):
    from decoding_step_amd.workloads import WORKLOADS
    nbytes, flops = bench.algorithmic_work(WORKLOADS["mixed_b16_l32"])
    M = 16 * 32
    w = 157184 * 2048 * 2
    h = M * 2048 * 2
    state = M * 15 + 2 * M * 4 * 8          # credit slots read and written (credit sequences present)
    assert nbytes == w + h + state == 645_963_264
    assert flops == 2 * M * 157184 * 2048 == 329_638_739_968
    # arithmetic intensity above the bf16 ridge (2.5 PFLOP/s / 8 TB/s = 312.5 flop/B): MFMA-bound
    assert flops / nbytes > 2500e12 / 8e12


def test_topk_adds_its_outputs(bench):
    from decoding_step_amd.workloads import WORKLOADS
    wl = WORKLOADS["threshold_b1_l32"]
    assert bench.algorithmic_work(wl, 8)[0] - bench.algorithmic_work(wl)[0] == 32 * 8 * 8


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
