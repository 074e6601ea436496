"""GPU parity of the bias gradient (jfa_backward's dbias) against the fp64 oracle.

The oracle's dbias is pinned by finite differences and by autograd of a dense reference
(test_oracle_backward.py). Tolerance: rel-L2 <= 2e-2, the gradient bound. Buckets that no visible
pair reaches must come out exactly 0, and so must the per-head scalar under softmax (its exact
gradient is 0: softmax is invariant to a shift of the whole row).
"""
import numpy as np
import pytest
import torch

import jfa_inputs as ji
from jagged_sequence_amd import binding as J
from oracle.bucket import bucket
from tests.gpu_util import GRAD_REL_L2, oracle, rel_l2, run_gpu, say, to_dev, to_np

pytestmark = pytest.mark.gpu

SELF_LENS = [1, 37, 130, 257]
CROSS_Q = [1, 37, 130, 64]
CROSS_KV = [5, 300, 64, 129]
MODES = [(D, m, a, b) for D in (64, 128) for m in ("none", "causal") for a in ("softmax", "silu", "gelu_tanh")
         for b in ("scalar", "bucket")]


def reached_buckets(x):
    """Buckets hit by at least one visible pair of any sequence (head independent)."""
    hit = np.zeros(64, dtype=bool)
    for b in range(len(x.q_off) - 1):
        lq, lkv = x.q_off[b + 1] - x.q_off[b], x.kv_off[b + 1] - x.kv_off[b]
        if lq == 0 or lkv == 0:
            continue
        i = np.arange(lq)[:, None]
        j = np.arange(lkv)[None, :]
        vis = np.ones((lq, lkv), dtype=bool) if x.mask == "none" else (j <= i)
        hit[np.unique(bucket(np.abs(i - j)[vis]))] = True
    return hit


def check_dbias(x, got, ref):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite dbias"
    if x.bias_kind == "scalar" and x.act == "softmax":
        assert np.all(got == 0.0), got
        return 0.0
    if x.bias_kind == "bucket":
        hit = reached_buckets(x)
        assert np.all(got[:, ~hit] == 0.0), "gradient in a bucket no visible pair reaches"
    err = float(rel_l2(got, ref))
    assert err <= GRAD_REL_L2, (err, got, ref)
    return err


@pytest.mark.parametrize("D,mask,act,bias", MODES, ids=["-".join(map(str, m)) for m in MODES])
def test_dbias_tiny_all_modes(D, mask, act, bias):
    lq, lkv = (SELF_LENS, SELF_LENS) if mask == "causal" else (CROSS_Q, CROSS_KV)
    x = ji.make_inputs(lq, lkv, 2, D, wid=42, mask=mask, act=act, bias_kind=bias, bias_sigma=0.5)
    say(f"case dbias D={D} mask={mask} act={act} bias={bias}")
    gpu = run_gpu(x, dbias=True)
    ref = oracle(x)
    err = check_dbias(x, to_np(gpu["dbias"]), ref["dbias"])
    say(f"  dbias rel-L2 {err:.2e}")


def test_dbias_deterministic_and_split_invariant():
    lens = [700, 129, 1, 300]
    x = ji.make_inputs(lens, lens, 2, 128, wid=43, mask="causal", act="softmax", bias_kind="bucket", bias_sigma=0.5)
    say("case dbias determinism / split")
    g0 = run_gpu(x, dbias=True, no_split=True)
    g0b = run_gpu(x, dbias=True, no_split=True)
    a, b = to_np(g0["dbias"]), to_np(g0b["dbias"])
    assert np.array_equal(a, b), "dbias differs between two identical runs"
    g1 = run_gpu(x, dbias=True, num_slots=16)
    assert len(g1["plan"].schedule(5)) > 0, "no dK/dV split at 16 slots"
    c = to_np(g1["dbias"])
    # Forcing 16 slots splits the forward too: its pieces round P to bf16 against their own running
    # maxima, so out and lse (hence Delta and dS) agree with the unsplit run to the bf16 operand
    # rounding (2^-8), as in the forward split test.
    assert float(np.abs(c - a).max()) <= 2.0 ** -8 * max(1.0, float(np.abs(a).max())), (a, c)
    check_dbias(x, c, oracle(x)["dbias"])


def test_dbias_requires_a_bias():
    """The binding refuses a bias gradient without a bias, and so does the library itself (called
    directly), before any launch."""
    import ctypes
    x = ji.make_inputs([40], [40], 1, 64, wid=44, mask="causal", act="softmax", bias_kind="none")
    say("case dbias without bias")
    with pytest.raises(ValueError, match="without bias"):
        run_gpu(x, dbias=True)
    g = run_gpu(x)
    plan = g["plan"]
    t = torch.zeros(64, dtype=torch.float32, device="cuda")
    p = lambda a: ctypes.c_void_p(a.data_ptr())
    q = to_dev(x.q)
    st = J.LIB.jfa_backward(plan._h, p(q), p(q), p(q), None, None, None, p(g["out"]), p(g["lse"]), p(q), p(g["dq"]),
                            p(g["dk"]), p(g["dv"]), p(t), None, 0, None)
    assert st == 4  # JFA_ERR_UNSUPPORTED


def test_dbias_full_causal_bucket_workload():
    """Full causal 64-bucket workload in the benchmark's launch configuration (bf16 outputs) against
    the oracle's dbias over the whole batch."""
    x = ji.workload_inputs("causal_bucket")
    say("case dbias workload causal_bucket (full batch)")
    gpu = run_gpu(x, out_dtype="bf16", grad_dtype="bf16", dbias=True)
    ref = oracle(x)
    err = check_dbias(x, to_np(gpu["dbias"]), ref["dbias"])
    say(f"  dbias rel-L2 {err:.2e}")


@pytest.mark.parametrize("act", ["softmax", "silu"])
@pytest.mark.parametrize("bias", ["scalar", "bucket"])
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_dbias_short_query_items(mask, bias, act):
    """Problems whose sequences all have at most 64 queries run the fused backward, which also
    accumulates the bias gradient."""
    lq, lkv = ([1, 37, 64, 50], [1, 37, 64, 50]) if mask == "causal" else ([1, 37, 64, 5], [300, 64, 129, 1000])
    x = ji.make_inputs(lq, lkv, 2, 128, wid=47, mask=mask, act=act, bias_kind=bias, bias_sigma=0.5)
    say(f"case dbias short-query mask={mask} bias={bias} act={act}")
    gpu = run_gpu(x, dbias=True)
    assert gpu["plan"].info()["fused_bwd"] == 1
    check_dbias(x, to_np(gpu["dbias"]), oracle(x)["dbias"])
