"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI, run the oracle, compare.

Tolerances (bf16 inputs, fp32 accumulation):
  forward output (fp32 store): max-abs <= 1e-2 and rel-L2 <= 5e-3; for GDPA rows of sequences with
      fewer than 100 keys each element may in addition differ by 2^-8 (1/Lkv) sum_j |act(s_ij)| |v_jd|,
      the rounding of the activation to a bf16 MFMA operand (GDPA outputs of such short sequences are
      not averaged; from 100 keys on, the shortest length of the GDPA workload, the plain 1e-2 holds
      and is asserted);
  forward output (bf16 store): rel-L2 <= 5e-3, every element within 1e-2 + half a bf16 ulp of |O|
      (rounding to bf16 alone can exceed 1e-2 once |O| >= 4);
  lse: max-abs <= 2e-3 (fp32 scores and sums; the only approximation is exp2/log2 at ~1 ulp);
  gradients: rel-L2 <= 2e-2.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import jfa_inputs as ji
from jagged_sequence_amd import binding as J
from oracle import attention as A

OUT_MAX_ABS = 1e-2
OUT_REL_L2 = 5e-3
LSE_MAX_ABS = 2e-3
GRAD_REL_L2 = 2e-2
GDPA_SHORT = 100  # shortest sequence of the GDPA workload


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_gpu(x: ji.Inputs, *, out_dtype="f32", grad_dtype="f32", num_slots=0, no_split=False, backward=True,
            scale=0.0, dbias=False):
    plan = J.Plan(x.q_off, x.kv_off, x.H, x.D, mask=x.mask, act=x.act, bias=x.bias_kind, out_dtype=out_dtype,
                  grad_dtype=grad_dtype, num_slots=num_slots, no_split=no_split, scale=scale, window=x.window,
                  block=x.block, shared_q=x.shared_q)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    qo = torch.from_numpy(x.q_off).cuda()
    ko = torch.from_numpy(x.kv_off).cuda()
    bias = torch.from_numpy(x.bias).cuda() if x.bias is not None else None
    out, lse = plan.forward(q, k, v, qo, ko, bias)
    res = {"plan": plan, "out": out, "lse": lse}
    if backward:
        do = to_dev(x.do)
        if dbias:
            dq, dk, dv, db = plan.backward(q, k, v, qo, ko, bias, out, lse, do, dbias=True)
            res["dbias"] = db
        else:
            dq, dk, dv = plan.backward(q, k, v, qo, ko, bias, out, lse, do)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return res


def oracle(x: ji.Inputs, *, backward=True, seqs=None, heads=None):
    f = A.bf16_bits_to_f64
    q, k, v = f(x.q), f(x.k), f(x.v)
    bias = None if x.bias is None else x.bias.astype(np.float64)
    kw = dict(mask=x.mask, act=x.act, bias_kind=x.bias_kind, bias=bias, seqs=seqs, heads=heads, window=x.window,
              block=x.block)
    if x.shared_q:  # the explicit copy of the shared rows for every sequence
        if seqs is not None:
            raise ValueError("shared queries: the query gradient sums over every sequence")
        q, _ = A.replicate_shared_q(q, x.B)
    out, lse = A.forward(q, k, v, x.q_off, x.kv_off, **kw)
    res = {"out": out, "lse": lse}
    if x.act != "softmax":
        res["mag"] = A.gdpa_magnitude(q, k, v, x.q_off, x.kv_off, **kw)
    if backward:
        if x.shared_q:
            dq, dk, dv, db = A.backward_shared_q(f(x.q), k, v, x.kv_off, f(x.do), **{k_: v_ for k_, v_ in kw.items()
                                                                                    if k_ != "seqs"})
        else:
            dq, dk, dv, db = A.backward(q, k, v, x.q_off, x.kv_off, f(x.do), **kw)
        res.update(dq=dq, dk=dk, dv=dv, dbias=db)
    return res


def rows_of(off, seqs):
    if seqs is None:
        return slice(None)
    return np.concatenate([np.arange(off[b], off[b + 1]) for b in seqs]).astype(np.int64)


def rel_l2(got, ref):
    n = np.linalg.norm(ref)
    d = np.linalg.norm(got - ref)
    return d / n if n > 0 else d


def compare(x: ji.Inputs, gpu, ref, *, seqs=None, heads=None, out_bf16=False, backward=True, plain=False):
    """Assert the tolerances on the selected sequences / heads; returns the error report.

    ``plain``: no GDPA operand-rounding term (workload-length sequences meet 1e-2 without it).
    """
    hsel = slice(None) if heads is None else list(heads)
    qr = rows_of(x.q_off, seqs)
    kr = rows_of(x.kv_off, seqs)
    rep = {}
    o_gpu = to_np(gpu["out"])[qr][:, hsel]
    o_ref = ref["out"][qr][:, hsel]
    err = np.abs(o_gpu - o_ref)
    rep["out_max_abs"] = float(err.max()) if err.size else 0.0
    rep["out_rel_l2"] = float(rel_l2(o_gpu, o_ref))
    assert np.all(np.isfinite(o_gpu)), "non-finite output"
    bound = np.full(err.shape, OUT_MAX_ABS)
    if "mag" in ref and not plain:
        # the operand-rounding allowance only for rows whose sequence has fewer than GDPA_SHORT keys
        lkv_row = np.repeat(np.diff(x.kv_off), np.diff(x.q_off))[qr]
        short = (lkv_row < GDPA_SHORT)[:, None, None]
        bound = bound + np.where(short, 2.0 ** -8 * ref["mag"][qr][:, hsel], 0.0)
    if out_bf16:
        bound = bound + np.exp2(np.floor(np.log2(np.maximum(np.abs(o_ref), 1e-30))) - 8)
    rep["out_worst_vs_bound"] = float((err / bound).max()) if err.size else 0.0
    assert np.all(err <= bound), rep
    assert rep["out_rel_l2"] <= OUT_REL_L2, rep
    if ref["lse"] is not None:
        l_gpu = to_np(gpu["lse"])[hsel][:, qr]
        l_ref = ref["lse"][hsel][:, qr]
        fin = np.isfinite(l_ref)
        assert np.array_equal(fin, np.isfinite(l_gpu)), "lse -inf pattern differs"
        rep["lse_max_abs"] = float(np.abs(l_gpu[fin] - l_ref[fin]).max()) if fin.any() else 0.0
        assert rep["lse_max_abs"] <= LSE_MAX_ABS, rep
    if backward:
        for name, rows in [("dq", slice(None) if x.shared_q else qr), ("dk", kr), ("dv", kr)]:
            g = to_np(gpu[name])[rows][:, hsel]
            r = ref[name][rows][:, hsel]
            assert np.all(np.isfinite(g)), f"non-finite {name}"
            rep[name + "_rel_l2"] = float(rel_l2(g, r))
            assert rep[name + "_rel_l2"] <= GRAD_REL_L2, rep
    return rep
