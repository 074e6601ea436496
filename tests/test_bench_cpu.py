"""Host legs of bench.py that need no GPU: the oracle timing (cpu_baseline) for every workload kind,
the --gpus guard and the algorithmic byte counts."""
import subprocess
import sys

import numpy as np
import pytest

import bench
import jfa_inputs as ji


def small_inputs(name):
    """A two-sequence stand-in with the workload's modes (the baseline only reads shapes and modes)."""
    w = ji.WORKLOADS[name]
    lq = [24, 24] if w.shared_q else [40, 17]
    lkv = [40, 17] if (w.kv_law is not None or w.shared_q) else lq
    if w.mask == "causal":
        lkv = lq
    return ji.make_inputs(lq, lkv, 2, w.D, wid=90, mask=w.mask, act=w.act, bias_kind=w.bias,
                          window=w.window, block=w.block, shared_q=bool(w.shared_q),
                          with_do=w.backward)


@pytest.mark.parametrize("name", sorted(ji.WORKLOADS))
def test_cpu_baseline_runs_for_every_workload(name):
    x = small_inputs(name)
    r = bench.cpu_baseline(x, name, seconds_target=0.01)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOPS"
    assert np.isfinite(r["value"]) and r["value"] > 0
    assert r["cores"] >= 1
    assert "sequences" in r["sample"]


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert p.returncode != 0
    assert "one GPU" in p.stderr


def test_kernel_bytes_counts_each_operand_once():
    # forward: Q, K, V read, O written (2 bytes each), lse written in fp32
    Tq, Tkv, H, D = 100, 300, 2, 128
    fwd = bench.kernel_bytes("forward", Tq, Tkv, H, D, out_bytes=2, softmax=True)
    assert fwd == 2 * H * D * (Tq + 2 * Tkv) + 2 * H * D * Tq + 4 * H * Tq


def test_kernel_bytes_mx_forward_reads_one_byte_and_a_scale():
    Tq, Tkv, H, D = 64, 64, 1, 128
    bf = bench.kernel_bytes("forward", Tq, Tkv, H, D, out_bytes=2, softmax=True)
    mx = bench.kernel_bytes("forward", Tq, Tkv, H, D, out_bytes=2, softmax=True, mx=True)
    # inputs: 3 x 64 x 128 elements, 2 bytes each against 1 + 1/32
    assert bf - mx == 3 * 64 * 128 * 2 - 3 * 64 * 128 * 33 // 32
