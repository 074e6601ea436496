"""Error paths of the C ABI on the GPU: every check runs before the first launch, so a rejected call
leaves every output untouched. Each case calls the library directly (the binding's own checks would
stop most of these earlier) with a canary pattern in the outputs."""
import ctypes
import os

import numpy as np
import pytest
import torch

import jfa_inputs as ji

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("no GPU", allow_module_level=True)

from jagged_sequence_amd import binding as J  # noqa: E402
from tests.gpu_util import say, to_dev  # noqa: E402

LENS = [300, 45, 700, 1]


def _setup(act="softmax"):
    x = ji.make_inputs(LENS, LENS, 2, 128, wid=60, mask="causal", act=act, bias_kind="bucket", bias_sigma=0.5)
    # few slots force split items, so both passes need a workspace
    plan = J.Plan(x.q_off, x.kv_off, 2, 128, mask="causal", act=act, bias="bucket", num_slots=32)
    fwd_ws, bwd_ws = plan.workspace_bytes()
    assert fwd_ws > 0 and bwd_ws > 0
    t = dict(q=to_dev(x.q), k=to_dev(x.k), v=to_dev(x.v), do=to_dev(x.do), bias=torch.from_numpy(x.bias).cuda(),
             qo=torch.from_numpy(x.q_off).cuda(), ko=torch.from_numpy(x.kv_off).cuda())
    Tq = x.q.shape[0]
    canary = lambda shape, dt: torch.full(shape, 7.0, dtype=dt, device="cuda")
    outs = dict(out=canary((Tq, 2, 128), torch.bfloat16), lse=canary((2, Tq), torch.float32),
                dq=canary((Tq, 2, 128), torch.bfloat16), dk=canary((Tq, 2, 128), torch.bfloat16),
                dv=canary((Tq, 2, 128), torch.bfloat16))
    ws = dict(f=torch.empty(fwd_ws, dtype=torch.uint8, device="cuda"), b=torch.empty(bwd_ws, dtype=torch.uint8,
                                                                                      device="cuda"))
    return plan, t, outs, ws


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _fwd(plan, t, o, ws, nbytes=None, q=None, qo="dev"):
    nb = ws.numel() if nbytes is None else nbytes
    off = (_p(t["qo"]), _p(t["ko"])) if qo == "dev" else qo
    return J.LIB.jfa_forward(plan._h, q if q is not None else _p(t["q"]), _p(t["k"]), _p(t["v"]), *off, _p(t["bias"]),
                             _p(o["out"]), _p(o["lse"]), _p(ws), nb, None)


def _bwd(plan, t, o, ws, nbytes=None, qo="dev"):
    nb = ws.numel() if nbytes is None else nbytes
    off = (_p(t["qo"]), _p(t["ko"])) if qo == "dev" else qo
    return J.LIB.jfa_backward(plan._h, _p(t["q"]), _p(t["k"]), _p(t["v"]), *off, _p(t["bias"]), _p(o["out"]),
                              _p(o["lse"]), _p(t["do"]), _p(o["dq"]), _p(o["dk"]), _p(o["dv"]), None, _p(ws), nb,
                              None)


def _untouched(o):
    torch.cuda.synchronize()
    for name, t in o.items():
        assert bool((t.float() == 7.0).all()), f"{name} was written by a rejected call"


def test_misaligned_tensor_is_rejected_before_any_launch():
    plan, t, o, ws = _setup()
    raw = torch.empty(t["q"].numel() + 8, dtype=torch.bfloat16, device="cuda")
    qmis = ctypes.c_void_p(raw.data_ptr() + 2)  # 2 bytes past a 16-byte boundary
    assert _fwd(plan, t, o, ws["f"], q=qmis) == 5  # JFA_ERR_MISALIGNED
    assert b"aligned" in J.LIB.jfa_last_error()
    wmis = ctypes.c_void_p(ws["b"].data_ptr() + 4)
    st = J.LIB.jfa_backward(plan._h, _p(t["q"]), _p(t["k"]), _p(t["v"]), _p(t["qo"]), _p(t["ko"]), _p(t["bias"]),
                            _p(o["out"]), _p(o["lse"]), _p(t["do"]), _p(o["dq"]), _p(o["dk"]), _p(o["dv"]), None,
                            wmis, ws["b"].numel() - 4, None)
    assert st == 5
    _untouched(o)
    say("misaligned pointers: JFA_ERR_MISALIGNED, outputs untouched")


def test_undersized_workspace_is_rejected_before_any_launch():
    plan, t, o, ws = _setup()
    assert _fwd(plan, t, o, ws["f"], nbytes=ws["f"].numel() - 256) == 6  # JFA_ERR_WORKSPACE
    assert _fwd(plan, t, o, None, nbytes=0) == 6
    assert _bwd(plan, t, o, ws["b"], nbytes=ws["b"].numel() - 256) == 6
    assert b"workspace" in J.LIB.jfa_last_error()
    _untouched(o)
    say("undersized workspace: JFA_ERR_WORKSPACE, outputs untouched")


def test_debug_offset_check(monkeypatch):
    """With JFA_DEBUG=1 the device offsets are compared with the planned ones (a synchronising
    check); a mismatch is JFA_ERR_BAD_OFFSETS before any launch, matching copies pass."""
    plan, t, o, ws = _setup()
    monkeypatch.setenv("JFA_DEBUG", "1")
    bad = t["qo"].clone()
    bad[2] += 1
    assert _fwd(plan, t, o, ws["f"], qo=(_p(bad), _p(t["ko"]))) == 2  # JFA_ERR_BAD_OFFSETS
    assert _bwd(plan, t, o, ws["b"], qo=(_p(t["qo"]), _p(bad))) == 2
    assert b"differ" in J.LIB.jfa_last_error()
    _untouched(o)
    # matching copies, and no copies at all (the check is then skipped), run normally
    assert _fwd(plan, t, o, ws["f"]) == 0
    assert _fwd(plan, t, o, ws["f"], qo=(None, None)) == 0
    assert _bwd(plan, t, o, ws["b"]) == 0
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o["dk"].float()).all()) and not bool((o["dk"].float() == 7.0).all())
    say("JFA_DEBUG offsets: mismatch rejected, matching copies accepted")


def test_plan_buffers_are_reused_only_after_the_device_is_done():
    """Plans built and destroyed while passes of earlier plans are still queued: each pass must see its
    own work lists (the cache hands a buffer out again only after its events completed)."""
    x = ji.make_inputs(LENS, LENS, 2, 128, wid=61, mask="causal", act="softmax", bias_kind="none")
    t = dict(q=to_dev(x.q), k=to_dev(x.k), v=to_dev(x.v))
    ref_plan = J.Plan(x.q_off, x.kv_off, 2, 128, mask="causal")
    ref, _ = ref_plan.forward(t["q"], t["k"], t["v"], None, None)
    torch.cuda.synchronize()
    outs = []
    side = torch.cuda.Stream()
    for i in range(6):
        # alternate a plan of this batch and one of a permuted batch, on two streams, destroying each
        perm = LENS[::-1] if i % 2 else LENS
        p_other = J.Plan(ji.offsets(perm), ji.offsets(perm), 2, 128, mask="causal", stream=side)
        p = J.Plan(x.q_off, x.kv_off, 2, 128, mask="causal")
        o, _ = p.forward(t["q"], t["k"], t["v"], None, None)
        outs.append(o)
        del p, p_other
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)
    say("plan buffer cache: 6 plans on two streams, every pass equal to the reference")
