"""GPU parity of the broadcast modes against the fp64 oracle, through the C ABI.

Shared queries (JFA_PLAN_SHARED_Q): one set of seed queries serves every sequence (pooling by
multihead attention); the oracle is the explicit replication, with the seed gradient summed over
sequences. Fused self + target: causal with more queries than keys, the rows past a user's history
being candidate rows that see the whole history.
"""
import numpy as np
import pytest
import torch

import jfa_inputs as ji

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("no GPU", allow_module_level=True)

from tests.gpu_util import compare, oracle, run_gpu, say, to_np  # noqa: E402

MODES = [(D, a, b) for D in (64, 128) for a in ("softmax", "silu", "gelu_tanh") for b in ("none", "scalar", "bucket")]


@pytest.mark.parametrize("D,act,bias", MODES, ids=["-".join(map(str, m)) for m in MODES])
@pytest.mark.parametrize("Ls", [5, 130])
def test_shared_queries(D, act, bias, Ls):
    lkv = [300, 1, 77, 129, 0, 64]
    x = ji.make_inputs([Ls] * len(lkv), lkv, 2, D, wid=80, mask="none", act=act, bias_kind=bias, bias_sigma=0.5,
                       shared_q=True)
    say(f"case shared queries Ls={Ls} D={D} act={act} bias={bias}")
    gpu = run_gpu(x)
    assert gpu["dq"].shape == (Ls, 2, D)
    # at most 64 shared rows (D = 128): the fused backward, its dQ pieces summed over sequences
    assert gpu["plan"].info()["fused_bwd"] == (1 if (D == 128 and Ls <= 64) else 0)
    rep = compare(x, gpu, oracle(x))
    say(f"  {rep}")


@pytest.mark.parametrize("act", ["softmax", "silu"])
def test_shared_queries_forced_split_and_bf16(act):
    lkv = [2000, 5, 700, 1]
    x = ji.make_inputs([40] * 4, lkv, 2, 128, wid=81, mask="none", act=act, bias_kind="bucket", shared_q=True)
    say(f"case shared queries split act={act}")
    g1 = run_gpu(x, num_slots=16)
    assert len(g1["plan"].schedule(1)) > 0  # split forward items
    ref = oracle(x)
    compare(x, g1, ref)
    g2 = run_gpu(x, out_dtype="bf16", grad_dtype="bf16")
    compare(x, g2, ref, out_bf16=True)
    # the seed gradient is summed in a fixed order: bit-identical on a repeat
    g3 = run_gpu(x, out_dtype="bf16", grad_dtype="bf16")
    assert torch.equal(g2["dq"], g3["dq"])


TARGET_MODES = [(D, a, b) for D in (64, 128) for a in ("softmax", "silu", "gelu_tanh")
                for b in ("none", "scalar", "bucket")]


@pytest.mark.parametrize("D,act,bias", TARGET_MODES, ids=["-".join(map(str, m)) for m in TARGET_MODES])
def test_fused_self_plus_target(D, act, bias):
    lh, lc = [130, 1, 257, 64, 5], [40, 3, 129, 1, 0]
    lq = [a + b for a, b in zip(lh, lc)]
    x = ji.make_inputs(lq, lh, 2, D, wid=82, mask="causal", act=act, bias_kind=bias, bias_sigma=0.5)
    say(f"case self+target D={D} act={act} bias={bias}")
    gpu = run_gpu(x)
    rep = compare(x, gpu, oracle(x))
    say(f"  {rep}")


@pytest.mark.parametrize("window", [0, 100])
def test_fused_self_plus_target_forced_split_and_window(window):
    lh, lc = [700, 129, 1, 300], [64, 200, 5, 1]
    lq = [a + b for a, b in zip(lh, lc)]
    x = ji.make_inputs(lq, lh, 2, 128, wid=83, mask="causal", act="softmax", bias_kind="bucket", window=window)
    say(f"case self+target split, window {window}")
    g = run_gpu(x, num_slots=16)
    if not window:  # (a window leaves every item shorter than the fair share: nothing to split)
        assert len(g["plan"].schedule(1)) > 0 and len(g["plan"].schedule(5)) > 0  # split forward and dK/dV items
    compare(x, g, oracle(x))


@pytest.mark.parametrize("name", ["self_target", "pma_seeds"])
def test_broadcast_workloads_full_size(name):
    """Both workloads at full size in the benchmark's launch configuration (bf16 outputs); the oracle on
    sampled sequences (fused pass) or on every sequence (shared queries: the seed gradient needs all)."""
    from tests.test_gpu_parity import _sub_inputs
    w = ji.WORKLOADS[name]
    x = ji.workload_inputs(name)
    say(f"case workload {name} full size")
    gpu = run_gpu(x, out_dtype="bf16", grad_dtype="bf16")
    if x.shared_q:
        rep = compare(x, gpu, oracle(x), out_bf16=True)
    else:
        lq, _ = ji.lengths(w)
        seqs = sorted({int(np.argmax(lq)), int(np.argmin(lq))} | set(np.random.default_rng(3).choice(w.B, 3, replace=False).tolist()))
        sub, qr, kr = _sub_inputs(x, seqs)
        g_sub = {"out": gpu["out"][qr], "lse": gpu["lse"][:, qr], "dq": gpu["dq"][qr], "dk": gpu["dk"][kr],
                 "dv": gpu["dv"][kr]}
        rep = compare(sub, g_sub, oracle(sub), out_bf16=True)
    say(f"  {rep}")
