"""The allocation-free backward entry point (jfa_backward_noalloc) against jfa_backward.

Both run the same kernels; the allocation-free one takes its workspace from the library's static
scratch array. Two calls in a row, the second with a smaller batch (the array keeps the first call's
contents), each compared with jfa_backward on the same inputs; then a plan too large for the array is
refused before any launch.
"""
import ctypes

import numpy as np
import pytest
import torch

import jfa_inputs as ji

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("no GPU", allow_module_level=True)

from jagged_sequence_amd import binding as J  # noqa: E402
from tests.gpu_util import say, to_dev  # noqa: E402

CASES = [
    # a batch with split items (few slots), bias gradient on
    dict(lens=[700, 129, 1, 300, 2048, 77], H=4, mask="causal", act="softmax", bias="bucket", slots=16, dbias=True),
    # a smaller batch next: the scratch array still holds the first call's partial sums and counters
    dict(lens=[5, 64, 200], H=2, mask="causal", act="silu", bias="scalar", slots=0, dbias=False),
]


def _run(case, wid):
    lens = case["lens"]
    x = ji.make_inputs(lens, lens, case["H"], 128, wid=wid, mask=case["mask"], act=case["act"],
                       bias_kind=case["bias"], bias_sigma=0.5)
    plan = J.Plan(x.q_off, x.kv_off, case["H"], 128, mask=case["mask"], act=case["act"], bias=case["bias"],
                  num_slots=case["slots"])
    assert plan.workspace_bytes()[1] <= J.NOALLOC_SCRATCH_BYTES
    q, k, v, do = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.do)
    bias = torch.from_numpy(x.bias).cuda()
    out, lse = plan.forward(q, k, v, None, None, bias)
    ref = plan.backward(q, k, v, None, None, bias, out, lse, do, dbias=True if case["dbias"] else None)
    got = [torch.full_like(t, 7.0) for t in ref[:3]]
    db = torch.full_like(ref[3], 7.0) if case["dbias"] else None
    res = J.jfa_backward_noalloc(plan, q, k, v, None, None, bias, out, lse, do, *got, dbias=db)
    torch.cuda.synchronize()
    return ref, res


def test_noalloc_backward_equals_backward_on_two_calls():
    for i, case in enumerate(CASES):
        say(f"case no-alloc call {i + 1}: lengths {case['lens']}, H {case['H']}, {case['act']}, {case['bias']}")
        ref, res = _run(case, 70 + i)
        for name, a, b in zip(["dq", "dk", "dv", "dbias"], ref, res):
            assert torch.equal(a, b), f"call {i + 1}: {name} differs from jfa_backward"
        say(f"  call {i + 1}: dq, dk, dv{', dbias' if case['dbias'] else ''} bitwise equal to jfa_backward")


def test_noalloc_refuses_a_workspace_beyond_the_scratch_array():
    # Delta alone needs H * Tq * 4 bytes: 16 heads x 1.2M rows = 76.8 MB > 64 MiB
    lens = [400_000] * 3
    plan = J.Plan(ji.offsets(lens), ji.offsets(lens), 16, 128, mask="causal")
    assert plan.workspace_bytes()[1] > J.NOALLOC_SCRATCH_BYTES
    buf = torch.full((1024,), 7.0, dtype=torch.float32, device="cuda")
    p = ctypes.c_void_p(buf.data_ptr())
    st = J.LIB.jfa_backward_noalloc(plan._h, p, p, p, None, None, None, p, p, p, p, p, p, None, None)
    assert st == 6, st  # JFA_ERR_WORKSPACE, before any launch
    assert b"scratch" in J.LIB.jfa_last_error()
    torch.cuda.synchronize()
    assert bool((buf == 7.0).all())
    say("  oversized plan refused with JFA_ERR_WORKSPACE, nothing written")
