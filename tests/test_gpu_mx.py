"""GPU parity of the MXFP8 forward (JFA_PLAN_MXFP8) against the MXFP8 oracle, through the C ABI, and
its numerics gate against the full-precision oracle.

Against ``oracle.mx`` (the same quantisation steps in fp64) the only differences are the device's
exp2 (about one ulp, which can move a probability across an E4M3 rounding midpoint) and fp32
accumulation. The scaled FP8 product does not accumulate exactly in fp32: the layout probe measured
its results within about 6e-5 of the exact sums, relative to their size, so scores differ from the
fp64 ones at that level and a small fraction of the probabilities round to the neighbouring E4M3
value. Bounds: output within 1e-2 plus 2^-3 of the element's magnitude (one such rounding flip),
rel-L2 <= 5e-3 (measured 1e-4 .. 2.5e-3), lse max-abs <= 2e-3. Against the full
precision oracle (no quantisation) the quantisation itself is the error: rel-L2 <= 0.1 (5.9% on
the oracle's own comparison, tests/test_oracle_mx.py)."""
import numpy as np
import pytest
import torch

import jfa_inputs as ji

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("no GPU", allow_module_level=True)

from jagged_sequence_amd import binding as J  # noqa: E402
from oracle import attention as A  # noqa: E402
from oracle import mx  # noqa: E402
from tests.gpu_util import rel_l2, say, to_dev, to_np  # noqa: E402

MX_OUT_REL = 5e-3
GATE_REL = 0.1


def _run(x, out_dtype="f32", num_slots=0):
    plan = J.Plan(x.q_off, x.kv_off, x.H, x.D, mask=x.mask, bias=x.bias_kind, out_dtype=out_dtype, num_slots=num_slots,
                  window=x.window, block=x.block, mxfp8=True)
    bias = torch.from_numpy(x.bias).cuda() if x.bias is not None else None
    out, lse = plan.forward(to_dev(x.q), to_dev(x.k), to_dev(x.v), None, None, bias)
    torch.cuda.synchronize()
    return plan, to_np(out), to_np(lse)


def _check(x, out, lse, rows=slice(None), out_bf16=False):
    f = A.bf16_bits_to_f64
    kw = dict(mask=x.mask, bias_kind=x.bias_kind, bias=None if x.bias is None else x.bias.astype(np.float64),
              window=x.window, block=x.block)
    ro, rl, mag = mx.forward(f(x.q), f(x.k), f(x.v), x.q_off, x.kv_off, magnitude=True, **kw)
    fo, _ = A.forward(f(x.q), f(x.k), f(x.v), x.q_off, x.kv_off, **kw)
    o, r, full = out[rows], ro[rows], fo[rows]
    err = np.abs(o - r)
    # one probability on the other side of an E4M3 rounding midpoint (device exp2 vs fp64) may move
    # an element by up to 2^-3 of its magnitude; such flips are rare (rel-L2 stays at 1e-4 .. 1e-3)
    bound = 1e-2 + 2.0 ** -3 * mag[rows] + (np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 1e-30))) - 8)
                                           if out_bf16 else 0.0)
    rep = {"out_max_abs": float(err.max()), "out_rel_l2": float(rel_l2(o, r)), "gate_rel_l2": float(rel_l2(o, full))}
    fin = np.isfinite(rl[:, rows])
    assert np.array_equal(fin, np.isfinite(lse[:, rows])), "lse -inf pattern differs"
    rep["lse_max_abs"] = float(np.abs(lse[:, rows][fin] - rl[:, rows][fin]).max()) if fin.any() else 0.0
    assert np.all(np.isfinite(o)), rep
    assert np.all(err <= bound), rep
    assert rep["out_rel_l2"] <= MX_OUT_REL, rep
    assert rep["lse_max_abs"] <= 2e-3, rep
    assert rep["gate_rel_l2"] <= GATE_REL, rep
    return rep


MODES = [(m, b, w) for m in ("none", "causal") for b in ("none", "scalar", "bucket") for w in (0, 100)]


@pytest.mark.parametrize("mask,bias,window", MODES, ids=["-".join(map(str, m)) for m in MODES])
def test_mx_forward_tiny(mask, bias, window):
    lq, lkv = ([1, 37, 130, 257], [1, 37, 130, 257]) if mask == "causal" else ([1, 37, 130, 64], [5, 300, 64, 129])
    x = ji.make_inputs(lq, lkv, 2, 128, wid=95, mask=mask, bias_kind=bias, bias_sigma=0.5, window=window)
    say(f"case mxfp8 mask={mask} bias={bias} window={window}")
    _, out, lse = _run(x)
    say(f"  {_check(x, out, lse)}")


def test_mx_forward_forced_split_and_bf16():
    lens = [700, 129, 1, 300]
    x = ji.make_inputs(lens, lens, 2, 128, wid=96, mask="causal", bias_kind="bucket")
    say("case mxfp8 split")
    plan, out, lse = _run(x, num_slots=16)
    assert len(plan.schedule(1)) > 0
    _check(x, out, lse)
    _, ob, lb = _run(x, out_dtype="bf16")
    _check(x, ob, lb, out_bf16=True)


def test_mx_plan_is_forward_only():
    x = ji.make_inputs([40], [40], 1, 128, wid=97, mask="causal")
    plan = J.Plan(x.q_off, x.kv_off, 1, 128, mask="causal", mxfp8=True)
    q = to_dev(x.q)
    out, lse = plan.forward(q, q, q, None, None)
    with pytest.raises(J.JfaError) as e:
        plan.backward(q, q, q, None, None, None, out, lse, q)
    assert e.value.status == 4
    for bad in [dict(act="silu"), dict(head_dim=64)]:
        with pytest.raises(J.JfaError):
            J.Plan(x.q_off, x.kv_off, 1, bad.get("head_dim", 128), act=bad.get("act", "softmax"), mxfp8=True)


def test_mx_forward_full_size_longtail():
    """The long-tail workload's MXFP8 forward at full size (bench configuration, bf16 output): whole
    sequences up to 2,048 tokens against the MXFP8 oracle, the 32,768-token ones through the gate on
    their first rows (a sequence's first rows only see its first keys)."""
    from tests.test_gpu_parity import _sub_inputs
    name = "longtail_mxfp8"
    w = ji.WORKLOADS[name]
    x = ji.workload_inputs(name)
    lq, _ = ji.lengths(w)
    say(f"case workload {name} full size")
    _, out, lse = _run(x, out_dtype="bf16")
    seqs = [int(b) for b in np.argsort(lq, kind="stable")[:1]] + [int(b) for b in np.flatnonzero(lq <= 2048)[[5, 77, -1]]]
    sub, qr, _ = _sub_inputs(x, seqs)
    qr = qr.cpu().numpy()
    rep = _check(sub, out[qr], lse[:, qr], out_bf16=True)
    say(f"  sampled sequences {rep}")
    # the first 1,024 rows of a 32,768-token sequence equal those of its 1,024-token prefix
    b = int(np.argmax(lq))
    pre = ji.make_inputs([1024], [1024], w.H, w.D, wid=0, mask=w.mask, bias_kind=w.bias)
    s = int(x.q_off[b])
    import dataclasses
    pre = dataclasses.replace(pre, q=x.q[s:s + 1024], k=x.k[s:s + 1024], v=x.v[s:s + 1024], bias=x.bias)
    rep = _check(pre, out[s:s + 1024], lse[:, s:s + 1024], out_bf16=True)
    say(f"  longest sequence, first 1,024 rows {rep}")
