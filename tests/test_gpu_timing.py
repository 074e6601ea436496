"""Per-kernel timing through the C ABI: records per launch, cleared and reused on re-enable, and
results unchanged by it."""
import numpy as np
import pytest
import torch

import jfa_inputs as ji

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("no GPU", allow_module_level=True)

from jagged_sequence_amd import binding as J  # noqa: E402
from tests.gpu_util import say, to_dev  # noqa: E402


def test_kernel_timing_records_and_reuse():
    lens = [300, 45, 128, 700]
    x = ji.make_inputs(lens, lens, 2, 128, wid=61, mask="causal", act="softmax", bias_kind="bucket", bias_sigma=0.5)
    say("case timing records")
    plan = J.Plan(x.q_off, x.kv_off, x.H, x.D, mask="causal", act="softmax", bias="bucket", num_slots=16)
    q, k, v, do = to_dev(x.q), to_dev(x.k), to_dev(x.v), to_dev(x.do)
    qo, ko = torch.from_numpy(x.q_off).cuda(), torch.from_numpy(x.kv_off).cuda()
    bias = torch.from_numpy(x.bias).cuda()

    def step():
        out, lse = plan.forward(q, k, v, qo, ko, bias)
        return (out, lse) + tuple(plan.backward(q, k, v, qo, ko, bias, out, lse, do))

    ref = step()
    torch.cuda.synchronize()
    plan.timing_enable(True)
    for _ in range(3):
        got = step()
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)  # timing does not change the results
    launched = {name: n for name, (ms, n) in ((nm, plan.timing_read(nm)) for nm in J.KERNELS)}
    for name in ("forward", "combine", "dq", "dkdv"):
        ms, n = plan.timing_read(name)
        assert n == 3 and 0.0 < ms < 1e4, (name, ms, n)
    # enabling again clears the records; the pooled events are reused
    plan.timing_enable(True)
    step()
    torch.cuda.synchronize()
    assert plan.timing_read("forward")[1] == 1 and plan.timing_read("dkdv")[1] == 1
    plan.timing_enable(False)
    step()
    torch.cuda.synchronize()
    assert plan.timing_read("forward")[1] == 0
    say(f"  launches over three steps: {launched}")
