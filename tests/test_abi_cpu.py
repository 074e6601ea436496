"""The C ABI on the CPU: exported symbols, host-only schedules vs the spec, argument checks.

No compute call is made here (no GPU): plans are built with JFA_PLAN_HOST_ONLY.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import jfa_inputs as ji
from oracle import schedule as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
B = pytest.importorskip("jagged_sequence_amd.binding", reason="libjfa.so not built")


def _declared():
    with open(os.path.join(ROOT, "include", "jfa.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:jfa_status|void|const char\*)\s+(jfa_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) == 12
    for n in names:
        assert hasattr(B.LIB, n), n
    assert sorted(B.SYMBOLS) == names


def test_status_strings():
    for code, name in B.STATUS_NAMES.items():
        assert B.LIB.jfa_status_string(code).decode() == name


def _host_plan(lq, lkv, H, D=128, **kw):
    return B.Plan(ji.offsets(lq), ji.offsets(lkv), H, D, host_only=True, **kw)


CASES = [
    ([5, 130, 0, 257, 64], [5, 130, 0, 257, 64], "causal"),
    ([1, 40, 3, 64, 0], [300, 17, 0, 1000, 9], "none"),
    ([700, 129, 1, 128, 256], [700, 129, 1, 128, 256], "causal"),
    ([2000], [2000], "causal"),
]


def _compare(plan, lq, lkv, H, causal, slots, split, window=0, block=0):
    info = plan.info()
    kw = dict(window=window, block=block)
    fi, fg, _ = S.query_tile_items(lq, lkv, H, causal, info["fwd_bm"], info["fwd_bn"], slots, split, **kw)
    qi, qg, _ = S.query_tile_items(lq, lkv, H, causal, info["dq_bm"], info["dq_bn"], slots, split, **kw)
    ki, kg, _ = S.key_tile_items(lq, lkv, H, causal, info["kv_bm"], info["kv_bn"], slots, split, **kw)
    for which, expect in enumerate([fi, fg, qi, qg, ki, kg]):
        got = plan.schedule(which)
        np.testing.assert_array_equal(got, np.array(expect, dtype=np.int32).reshape(got.shape), err_msg=str(which))
    for which, lst in [(6, fi), (7, qi), (8, ki)]:
        got = plan.schedule(which)
        expect = S.dispatch_order(lst)
        np.testing.assert_array_equal(got, np.array(expect, dtype=np.int32).reshape(got.shape), err_msg=str(which))


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("slots", [1, 3, 64, 512])
@pytest.mark.parametrize("split", [True, False])
def test_schedule_bit_exact_vs_spec(case, slots, split):
    lq, lkv, mask = CASES[case]
    plan = _host_plan(lq, lkv, 3, mask=mask, num_slots=slots, no_split=not split)
    assert plan.info()["fwd_slots"] == slots
    _compare(plan, lq, lkv, 3, mask == "causal", slots, split)


BAND_CASES = [
    ([5, 130, 0, 257, 64, 700], [5, 130, 0, 257, 64, 700], "causal", 100, 0),
    ([5, 130, 0, 257, 64, 700], [5, 130, 0, 257, 64, 700], "causal", 1, 0),
    ([5, 130, 0, 257, 64, 700], [5, 130, 0, 257, 64, 700], "causal", 0, 200),
    ([5, 130, 0, 257, 64, 700], [5, 130, 0, 257, 64, 700], "causal", 300, 256),
    ([1, 40, 3, 64, 300], [300, 17, 0, 1000, 90], "none", 70, 0),
    ([1, 40, 3, 64, 300], [300, 17, 0, 1000, 90], "none", 0, 50),
    ([700, 129, 1], [700, 129, 1], "none", 64, 128),
    ([40, 3, 64], [40, 3, 64], "none", 0, 16),
]


@pytest.mark.parametrize("case", range(len(BAND_CASES)))
@pytest.mark.parametrize("slots", [1, 7, 512])
@pytest.mark.parametrize("D", [64, 128])
def test_band_schedule_bit_exact_vs_spec(case, slots, D):
    """Window / block limits: the planner's lists equal the spec's, including empty ranges."""
    lq, lkv, mask, window, block = BAND_CASES[case]
    plan = _host_plan(lq, lkv, 2, D=D, mask=mask, num_slots=slots, window=window, block=block)
    _compare(plan, lq, lkv, 2, mask == "causal", slots, True, window, block)


@pytest.mark.parametrize("name", ["small_fwd", "causal_bucket", "target_attn", "gdpa_silu", "longtail"])
def test_workload_schedules_bit_exact(name):
    w = ji.WORKLOADS[name]
    lq, lkv = ji.lengths(w)
    plan = _host_plan(lq, lkv, w.H, w.D, mask=w.mask, act=w.act, bias=w.bias)
    assert plan.info()["fwd_slots"] == 512
    _compare(plan, lq, lkv, w.H, w.mask == "causal", 512, True)


@pytest.mark.parametrize("name", ["causal_bucket", "longtail"])
def test_dispatch_order_keeps_groups_on_one_xcd(name):
    """Dispatch order: a permutation of the list; position p runs on XCD p % 8; away from the tail
    (where drained queues lend positions) every (b, h) group sits on a single XCD, and the XCD loads
    differ by less than the largest group."""
    w = ji.WORKLOADS[name]
    lq, lkv = ji.lengths(w)
    plan = _host_plan(lq, lkv, w.H, w.D, mask=w.mask, act=w.act, bias=w.bias)
    for lw, dw in [(0, 6), (2, 7), (4, 8)]:
        lst, disp = plan.schedule(lw), plan.schedule(dw)
        key = lambda a: sorted(map(tuple, a.tolist()))
        assert key(lst) == key(disp)
        n = len(disp)
        home = {}
        body = n - 8 * 8  # positions before the last rounds
        for p in range(max(0, body)):
            b, h = int(disp[p][0]), int(disp[p][1])
            assert home.setdefault((b, h), p % 8) == p % 8, (b, h)
        gsize = {}
        for b, h, _t, lo, hi, _s in lst.tolist():
            gsize[(b, h)] = gsize.get((b, h), 0) + hi - lo
        tot = [0] * 8
        for p in range(n):
            tot[p % 8] += disp[p][4] - disp[p][3]
        assert max(tot) - min(tot) <= max(gsize.values()) + max(1, sum(gsize.values()) // 100)


def test_short_query_problems_use_half_width_key_items():
    # softmax, D = 128 and every sequence with at most 64 queries: 64-key dK/dV items
    assert _host_plan([1, 64, 30], [500, 64, 7], 2, 128, mask="none").info()["kv_bn"] == 64
    assert _host_plan([1, 64, 30], [1, 64, 30], 2, 128, mask="causal").info()["kv_bn"] == 64
    assert _host_plan([1, 65, 30], [500, 65, 7], 2, 128, mask="none").info()["kv_bn"] == 128
    assert _host_plan([1, 64, 30], [500, 64, 7], 2, 128, mask="none", act="silu").info()["kv_bn"] == 128
    assert _host_plan([1, 64, 30], [500, 64, 7], 2, 64, mask="none").info()["kv_bn"] == 128
    w = ji.WORKLOADS["target_attn"]
    lq, lkv = ji.lengths(w)
    assert _host_plan(lq, lkv, w.H, w.D, mask=w.mask, act=w.act, bias=w.bias).info()["kv_bn"] == 64


def test_fused_backward_eligibility():
    """The backward runs as one fused pass over the dQ items exactly when those items cover every
    key: short query sets (D = 128, any activation, shared queries too), no window or block limit,
    and no sequence that has keys but no queries."""
    fused = lambda *a, **kw: _host_plan(*a, **kw).info()["fused_bwd"]
    assert fused([1, 64, 30], [500, 64, 7], 2, 128, mask="none") == 1
    assert fused([1, 64, 30], [1, 64, 30], 2, 128, mask="causal") == 1
    assert fused([1, 0, 30], [500, 0, 7], 2, 128, mask="none") == 1      # empty sequence
    assert fused([1, 0, 30], [500, 64, 7], 2, 128, mask="none") == 0     # keys without queries
    assert fused([1, 64, 30], [500, 64, 7], 2, 128, mask="none", window=16) == 0
    assert fused([1, 64, 30], [500, 64, 7], 2, 128, mask="none", act="silu") == 1
    assert fused([1, 65, 30], [500, 65, 7], 2, 128, mask="none") == 0
    assert fused([1, 64, 30], [500, 64, 7], 2, 64, mask="none") == 0
    assert fused([32, 32, 32], [500, 64, 7], 2, 128, mask="none", shared_q=True) == 1
    assert fused([65, 65, 65], [500, 64, 7], 2, 128, mask="none", shared_q=True) == 0
    w = ji.WORKLOADS["target_attn"]
    lq, lkv = ji.lengths(w)
    assert fused(lq, lkv, w.H, w.D, mask=w.mask, act=w.act, bias=w.bias) == 1


def test_workspace_sizes():
    lq = [700, 129, 1]
    plan = _host_plan(lq, lq, 2, mask="causal", num_slots=16)
    fwd, bwd = plan.workspace_bytes()
    nf = sum(R for (*_g, R) in plan.schedule(1))
    nq = sum(R for (*_g, R) in plan.schedule(3))
    nk = sum(R for (*_g, R) in plan.schedule(5))
    al = lambda x: (x + 255) // 256 * 256
    assert nf > 0 and nq > 0 and nk > 0
    assert fwd == al(nf * 128 * 128 * 4) + al(nf * 128 * 4)
    # Delta, dQ partials, dK and dV partials, and (D = 128) the dK/dV work-queue counters
    assert bwd == al(2 * 830 * 4) + al(nq * 128 * 128 * 4) + 2 * al(nk * 128 * 128 * 4) + al(8 * 4)
    plan2 = _host_plan(lq, lq, 2, mask="causal", num_slots=4, no_split=True, act="silu")
    assert plan2.workspace_bytes() == (0, al(8 * 4))
    plan3 = _host_plan(lq, lq, 2, 64, mask="causal", num_slots=4, no_split=True, act="silu")
    assert plan3.workspace_bytes() == (0, 0)


def _status_of(fn):
    with pytest.raises(B.JfaError) as e:
        fn()
    return B.STATUS_NAMES[e.value.status]


def test_plan_validation_errors():
    ok = ([3, 4], [3, 4])
    assert _status_of(lambda: _host_plan(*ok, 2, D=96)) == "JFA_ERR_BAD_SHAPE"
    assert _status_of(lambda: _host_plan(*ok, 0)) == "JFA_ERR_BAD_SHAPE"
    assert _status_of(lambda: B.Plan([0], [0], 2, 64, host_only=True)) == "JFA_ERR_BAD_SHAPE"
    assert _status_of(lambda: B.Plan([1, 3], [0, 3], 2, 64, host_only=True)) == "JFA_ERR_BAD_OFFSETS"
    assert _status_of(lambda: B.Plan([0, 3, 2], [0, 3, 4], 2, 64, host_only=True)) == "JFA_ERR_BAD_OFFSETS"
    assert _status_of(lambda: _host_plan([3, 4], [3, 5], 2, mask="causal")) == "JFA_ERR_BAD_SHAPE"
    assert _status_of(lambda: _host_plan(*ok, 2, num_slots=-1)) == "JFA_ERR_BAD_SHAPE"
    assert _status_of(lambda: _host_plan(*ok, 2, scale=float("nan"))) == "JFA_ERR_UNSUPPORTED"
    assert _status_of(lambda: _host_plan(*ok, 2, window=-1)) == "JFA_ERR_BAD_SHAPE"
    assert _status_of(lambda: _host_plan(*ok, 2, block=-3)) == "JFA_ERR_BAD_SHAPE"
    # causal with equal lengths and an empty sequence is fine
    _host_plan([3, 0, 4], [3, 0, 4], 2, mask="causal")


def test_raw_abi_null_and_enum_errors():
    lib = B.LIB
    h = ctypes.c_void_p()
    assert lib.jfa_plan(None, None, ctypes.byref(h)) == 1  # JFA_ERR_NULL_ARG
    off = np.array([0, 3], dtype=np.int32)
    p = B.Problem()
    p.num_seqs, p.num_heads, p.head_dim = 1, 1, 64
    p.q_offsets_host = off.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    p.kv_offsets_host = None
    p.flags = B.PLAN_HOST_ONLY
    assert lib.jfa_plan(ctypes.byref(p), None, ctypes.byref(h)) == 1
    p.kv_offsets_host = off.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    for field, bad in [("mask", 2), ("act", 3), ("bias", 7), ("out_dtype", 2)]:
        setattr(p, field, bad)
        assert lib.jfa_plan(ctypes.byref(p), None, ctypes.byref(h)) == 4, field  # UNSUPPORTED
        setattr(p, field, 0)
    p.flags = B.PLAN_HOST_ONLY | 0x80
    assert lib.jfa_plan(ctypes.byref(p), None, ctypes.byref(h)) == 4
    p.flags = B.PLAN_HOST_ONLY
    assert lib.jfa_plan(ctypes.byref(p), None, ctypes.byref(h)) == 0
    # a host-only plan refuses to launch, before touching any pointer
    assert lib.jfa_forward(h, *([None] * 8), None, 0, None) == 8
    assert b"host-only" in lib.jfa_last_error()
    assert lib.jfa_backward(h, *([None] * 13), None, 0, None) == 8
    assert lib.jfa_forward(None, *([None] * 8), None, 0, None) == 1
    lib.jfa_plan_destroy(h)
    lib.jfa_plan_destroy(None)


def test_negative_scale_rejected():
    # A negative multiplier would turn the -inf of a masked score into the row maximum.
    assert _status_of(lambda: _host_plan([3, 4], [3, 4], 2, scale=-0.5)) == "JFA_ERR_UNSUPPORTED"
    assert _status_of(lambda: _host_plan([3, 4], [3, 4], 2, scale=float("inf"))) == "JFA_ERR_UNSUPPORTED"
    _host_plan([3, 4], [3, 4], 2, scale=0.25)


def test_slice_limit_for_32bit_addressing():
    # (L + 128) * H * D <= 2^30: with H = 64, D = 128 the longest sequence may hold 130,944 rows.
    H, D = 64, 128
    L = (1 << 30) // (H * D) - 128
    _host_plan([L], [L], H, D, no_split=True)
    assert _status_of(lambda: _host_plan([L + 1], [L + 1], H, D)) == "JFA_ERR_BAD_SHAPE"
    assert _status_of(lambda: _host_plan([5, 3], [5, L + 1], H, D)) == "JFA_ERR_BAD_SHAPE"
    assert b"2^30" in B.LIB.jfa_last_error()


def _cpu_tensors(plan, out_dtype="bf16", grad_dtype="bf16"):
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    t = dict(q=torch.zeros(plan.Tq, plan.H, plan.D, dtype=bf), k=torch.zeros(plan.Tkv, plan.H, plan.D, dtype=bf),
             v=torch.zeros(plan.Tkv, plan.H, plan.D, dtype=bf), dout=torch.zeros(plan.Tq, plan.H, plan.D, dtype=bf),
             out=torch.zeros(plan.Tq, plan.H, plan.D, dtype=f32 if out_dtype == "f32" else bf),
             lse=torch.zeros(plan.H, plan.Tq, dtype=f32),
             bias=torch.zeros(plan.H, 64, dtype=f32) if plan.bias_kind == "bucket" else None)
    return t


def test_binding_checks_every_tensor_before_the_call():
    """Shape, dtype, layout and device of each tensor are checked in the binding (the library only sees
    pointers); CPU tensors reach the device check last, so each mismatch below is caught first."""
    import torch
    plan = _host_plan([5, 9], [5, 9], 2, mask="causal", bias="bucket")
    t = _cpu_tensors(plan)
    fwd = lambda **kw: plan.forward(kw.get("q", t["q"]), kw.get("k", t["k"]), kw.get("v", t["v"]), None, None,
                                    kw.get("bias", t["bias"]), out=kw.get("out"), lse=kw.get("lse"))
    bwd = lambda **kw: plan.backward(t["q"], t["k"], t["v"], None, None, t["bias"], kw.get("out", t["out"]),
                                     kw.get("lse", t["lse"]), kw.get("dout", t["dout"]), dq=kw.get("dq"),
                                     dk=kw.get("dk"), dv=kw.get("dv"), dbias=kw.get("dbias"))
    cases = [
        (fwd, dict(q=t["q"][:-1]), "shape"),
        (fwd, dict(k=t["k"].float()), "dtype"),
        (fwd, dict(v=t["v"].transpose(0, 1).contiguous().transpose(0, 1)), "contiguous"),
        (fwd, dict(bias=t["bias"][:, :32]), "shape"),
        (fwd, dict(bias=None), "required"),
        (fwd, dict(out=torch.zeros(14, 2, 128, dtype=torch.float32)), "dtype"),
        (fwd, dict(lse=torch.zeros(14, 2)), "shape"),
        (bwd, dict(dout=t["dout"].float()), "dtype"),
        (bwd, dict(dq=torch.zeros(14, 2, 128, dtype=torch.float32)), "dtype"),
        (bwd, dict(dk=torch.zeros(13, 2, 128, dtype=torch.bfloat16)), "shape"),
        (bwd, dict(out=None), "required"),
        (bwd, dict(dbias=torch.zeros(2, 63)), "shape"),
        (fwd, dict(), "GPU tensor"),
        (bwd, dict(), "GPU tensor"),
    ]
    for fn, kw, what in cases:
        with pytest.raises(ValueError, match=what):
            fn(**kw)
    nob = _host_plan([5], [7], 2)
    t2 = _cpu_tensors(nob)
    with pytest.raises(ValueError, match="without bias"):
        nob.forward(t2["q"], t2["k"], t2["v"], None, None, torch.zeros(2, 64))


def test_fused_self_target_lists_match_spec():
    """Causal with more queries than keys (target rows past the history): the lists follow the same
    rules; fewer queries than keys is refused."""
    lh, lc = [130, 5, 700, 64], [40, 0, 129, 200]
    lq = [a + b for a, b in zip(lh, lc)]
    for slots, split in [(512, True), (16, True), (16, False)]:
        plan = _host_plan(lq, lh, 2, mask="causal", num_slots=slots, no_split=not split)
        _compare(plan, lq, lh, 2, True, slots, split)
    assert _status_of(lambda: _host_plan([3, 4], [3, 5], 2, mask="causal")) == "JFA_ERR_BAD_SHAPE"


def test_shared_query_dq_groups_match_spec():
    """Shared queries: every dQ piece gets a partial slot and one group per (head, query tile) sums the
    pieces of all sequences; the forward and dK/dV lists are unchanged."""
    Ls, lkv = 150, [300, 1, 77, 1000, 0]
    lq = [Ls] * len(lkv)
    for slots, split in [(512, True), (8, True)]:
        plan = B.Plan(ji.offsets(lq), ji.offsets(lkv), 2, 128, host_only=True, num_slots=slots, no_split=not split,
                      shared_q=True)
        info = plan.info()
        qi, _, _ = S.query_tile_items(lq, lkv, 2, False, info["dq_bm"], info["dq_bn"], slots, split)
        items, groups, n = S.share_query_slots(qi)
        np.testing.assert_array_equal(plan.schedule(2), np.array(items, dtype=np.int32).reshape(-1, 6))
        np.testing.assert_array_equal(plan.schedule(3), np.array(groups, dtype=np.int32).reshape(-1, 5))
        assert sorted(g[2] for g in groups) == [0, 0, 1, 1] and sum(g[4] for g in groups) == len(items)
        fi, fg, _ = S.query_tile_items(lq, lkv, 2, False, info["fwd_bm"], info["fwd_bn"], slots, split)
        np.testing.assert_array_equal(plan.schedule(0), np.array(fi, dtype=np.int32).reshape(-1, 6))
    assert _status_of(lambda: B.Plan(ji.offsets([3, 4]), ji.offsets([3, 4]), 2, 64, host_only=True,
                                     shared_q=True)) == "JFA_ERR_BAD_SHAPE"
