"""GPU parity of the window / block masks (through the C ABI) against the fp64 oracle.

The oracle's band visibility is pinned in test_oracle_band.py (torch attention with the band as an
additive mask, block attention as attention on the cut sequences, window 1, finite differences).
Tolerances are those of every other parity test (tests/gpu_util.py).
"""
import numpy as np
import pytest
import torch

import jfa_inputs as ji

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("no GPU", allow_module_level=True)

from tests.gpu_util import GRAD_REL_L2, compare, oracle, rel_l2, run_gpu, say, to_np  # noqa: E402

# self-attention lengths spanning several 64/128 tiles with ragged tails; cross lengths where some
# query rows see no key at all under a window or block (rows far past the last key)
SELF_LENS = [1, 37, 130, 257, 700]
CROSS_Q = [1, 37, 130, 64, 300]
CROSS_KV = [5, 300, 64, 129, 90]
# (mask, window, block)
BANDS = [("causal", 100, 0), ("causal", 1, 0), ("causal", 0, 96), ("causal", 200, 128),
         ("none", 70, 0), ("none", 0, 50), ("none", 64, 128)]
BIASES = ("none", "scalar", "bucket")
CASES = [(D, act, bi, BIASES[(bi + ai + D // 64) % 3]) for D in (64, 128)
         for ai, act in enumerate(("softmax", "silu", "gelu_tanh")) for bi in range(len(BANDS))]


def _inputs(D, act, band, bias, wid=50, H=2):
    mask, window, block = band
    lq, lkv = (SELF_LENS, SELF_LENS) if mask == "causal" else (CROSS_Q, CROSS_KV)
    return ji.make_inputs(lq, lkv, H, D, wid=wid, mask=mask, act=act, bias_kind=bias, bias_sigma=0.5,
                          window=window, block=block)


@pytest.mark.parametrize("D,act,bi,bias", CASES, ids=[f"D{c[0]}-{c[1]}-band{c[2]}-{c[3]}" for c in CASES])
def test_band_tiny(D, act, bi, bias):
    x = _inputs(D, act, BANDS[bi], bias)
    say(f"case band D={D} act={act} band={BANDS[bi]} bias={bias}")
    gpu = run_gpu(x)
    rep = compare(x, gpu, oracle(x))
    say(f"  {rep}")


@pytest.mark.parametrize("act", ["softmax", "silu"])
def test_band_forced_split(act):
    x = _inputs(128, act, ("causal", 300, 0), "bucket", wid=51)
    say(f"case band split act={act}")
    gpu = run_gpu(x, num_slots=64)
    plan = gpu["plan"]
    assert len(plan.schedule(1)) > 0 and len(plan.schedule(3)) > 0 and len(plan.schedule(5)) > 0
    compare(x, gpu, oracle(x))


def test_band_rows_with_no_visible_key():
    # block 32 with Lq far past Lkv: query rows in blocks that hold no key see nothing
    x = ji.make_inputs([100, 70], [20, 3], 2, 128, wid=52, mask="none", act="softmax", bias_kind="scalar",
                       block=32)
    say("case band empty rows")
    gpu = run_gpu(x)
    ref = oracle(x)
    assert np.all(np.isneginf(to_np(gpu["lse"])[:, 32:100]))
    assert np.all(to_np(gpu["out"])[32:100] == 0.0) and np.all(to_np(gpu["dq"])[32:100] == 0.0)
    compare(x, gpu, ref)


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0)])
def test_band_short_query_items(mask, window):
    """Lq <= 64 everywhere (half-width dK/dV items) with a block / window limit."""
    lq, lkv = ([1, 37, 64, 50], [1, 37, 64, 50]) if mask == "causal" else ([1, 37, 64, 5], [300, 64, 129, 1000])
    x = ji.make_inputs(lq, lkv, 2, 128, wid=53, mask=mask, act="softmax", bias_kind="bucket", window=window or 20,
                       block=48)
    say(f"case band short-query mask={mask}")
    gpu = run_gpu(x)
    assert gpu["plan"].info()["kv_bn"] == 64
    compare(x, gpu, oracle(x))


@pytest.mark.parametrize("D,act", [(128, "softmax"), (128, "silu"), (64, "softmax")])
def test_band_dbias(D, act):
    x = _inputs(D, act, ("causal", 200, 128), "bucket", wid=54)
    say(f"case band dbias D={D} act={act}")
    gpu = run_gpu(x, dbias=True)
    ref = oracle(x)
    compare(x, gpu, ref)
    err = float(rel_l2(to_np(gpu["dbias"]), ref["dbias"]))
    say(f"  dbias rel-L2 {err:.2e}")
    assert err <= GRAD_REL_L2


SHORT_DBIAS = [("none", [1, 37, 64, 5], [300, 64, 129, 1000], 20, 48),
               ("causal", [1, 37, 64, 50], [1, 37, 64, 50], 20, 48),
               ("none", [0, 30, 64], [50, 40, 129], 0, 0)]


@pytest.mark.parametrize("mask,lq,lkv,window,block", SHORT_DBIAS, ids=["band", "band-causal", "keys-without-queries"])
def test_short_query_items_dbias(mask, lq, lkv, window, block):
    """Half-width dK/dV items (two barriers per tile; used when the fused short-query pass is not
    eligible) with the bias gradient, whose bucket ids come from the score wave's bias window."""
    x = ji.make_inputs(lq, lkv, 2, 128, wid=55, mask=mask, act="softmax", bias_kind="bucket", bias_sigma=0.5,
                       window=window, block=block)
    say(f"case short-query dbias mask={mask} window={window} block={block} lq={lq}")
    gpu = run_gpu(x, dbias=True)
    info = gpu["plan"].info()
    assert info["kv_bn"] == 64 and info["fused_bwd"] == 0
    ref = oracle(x)
    compare(x, gpu, ref)
    err = float(rel_l2(to_np(gpu["dbias"]), ref["dbias"]))
    say(f"  dbias rel-L2 {err:.2e}")
    assert err <= GRAD_REL_L2


def _sample(lq, cap, n_random, seed):
    """The longest sequence no longer than ``cap``, the shortest, and ``n_random`` random ones."""
    order = [int(b) for b in np.argsort(lq, kind="stable")]
    longest = max((b for b in order if lq[b] <= cap), key=lambda b: lq[b])
    rng = np.random.default_rng(seed)
    pick = {longest, order[0]} | set(rng.choice(len(lq), size=n_random, replace=False).tolist())
    return sorted(int(b) for b in pick)


def test_full_size_sliding_window_sampled():
    """The long-tail sliding-window workload at full size, in the benchmark's launch configuration;
    the oracle checks sampled sequences on two heads."""
    name = "longtail_swa"
    x = ji.workload_inputs(name)
    lq, _ = ji.lengths(ji.WORKLOADS[name])
    seqs = _sample(lq, 8192, 2, 11)
    say(f"case workload {name} seqs={seqs} lengths={[int(lq[b]) for b in seqs]}")
    gpu = run_gpu(x, out_dtype="bf16", grad_dtype="bf16")
    heads = [0, 5]
    ref = oracle(x, seqs=seqs, heads=heads)
    rep = compare(x, gpu, ref, seqs=seqs, heads=heads, out_bf16=True, plain=True)
    say(f"  {rep}")
