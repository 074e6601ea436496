"""Pins of the oracle's backward pass (CPU): finite differences, library autograd, invariants."""
import math

import numpy as np
import pytest

import jfa_inputs as ji
from oracle import attention as A
from tests.oracle_pins_util import dense_gdpa, dense_softmax

MODES = [(m, a, b) for m in ["none", "causal"] for a in ["softmax", "silu", "gelu_tanh"]
         for b in ["none", "scalar", "bucket"]]


def _case(lq, lkv, H, D, wid, mask, act, bias_kind):
    x = ji.make_inputs(lq, lkv, H, D, wid=wid, mask=mask, act=act, bias_kind=bias_kind, bias_sigma=0.5)
    f = A.bf16_bits_to_f64
    bias = None if x.bias is None else x.bias.astype(np.float64)
    return x, f(x.q), f(x.k), f(x.v), f(x.do), bias


def _loss(q, k, v, x, do, mask, act, bias_kind, bias):
    out, _ = A.forward(q, k, v, x.q_off, x.kv_off, mask=mask, act=act, bias_kind=bias_kind, bias=bias)
    return float((out * do).sum())


def _fd(fn, arr, h=1e-6):
    g = np.zeros_like(arr)
    flat = arr.reshape(-1)
    gf = g.reshape(-1)
    for n in range(flat.size):
        old = flat[n]
        flat[n] = old + h
        up = fn()
        flat[n] = old - h
        dn = fn()
        flat[n] = old
        gf[n] = (up - dn) / (2 * h)
    return g


@pytest.mark.parametrize("mask,act,bias_kind", MODES)
def test_gradients_match_finite_differences(mask, act, bias_kind):
    lq, lkv = ([3, 5, 1], [3, 5, 1]) if mask == "causal" else ([3, 2, 1], [4, 1, 6])
    x, q, k, v, do, bias = _case(lq, lkv, 2, 4, 11, mask, act, bias_kind)
    dq, dk, dv, db = A.backward(q, k, v, x.q_off, x.kv_off, do, mask=mask, act=act, bias_kind=bias_kind,
                                bias=bias)
    fn = lambda: _loss(q, k, v, x, do, mask, act, bias_kind, bias)
    for got, arr in [(dq, q), (dk, k), (dv, v)] + ([(db, bias)] if bias is not None else []):
        ref = _fd(fn, arr)
        # the softmax gradient of a per-head scalar bias is exactly 0: bound the denominator
        err = np.linalg.norm(got - ref) / max(1e-2, np.linalg.norm(ref))
        assert err < 1e-7, err


@pytest.mark.parametrize("mask,act,bias_kind", MODES)
def test_gradients_match_library_autograd(mask, act, bias_kind):
    lq, lkv = ([9, 17, 2, 6], [9, 17, 2, 6]) if mask == "causal" else ([9, 17, 2, 6], [12, 3, 20, 1])
    x, q, k, v, do, bias = _case(lq, lkv, 2, 16, 12, mask, act, bias_kind)
    scale = 1 / math.sqrt(16)
    dq, dk, dv, db = A.backward(q, k, v, x.q_off, x.kv_off, do, mask=mask, act=act, bias_kind=bias_kind,
                                bias=bias)
    if act == "softmax":
        _, _, rq, rk, rv, rb = dense_softmax(q, k, v, x.q_off, x.kv_off, mask, bias_kind, bias, scale,
                                             want_grad=True, dout=do)
    else:
        _, rq, rk, rv, rb = dense_gdpa(q, k, v, x.q_off, x.kv_off, mask, act, bias_kind, bias, scale,
                                       want_grad=True, dout=do)
    for got, ref in [(dq, rq), (dk, rk), (dv, rv)] + ([(db, rb)] if bias is not None else []):
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)


@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("bias_kind", ["none", "scalar", "bucket"])
def test_softmax_invariants(mask, bias_kind):
    lens = [13, 4, 21]
    lkv = lens if mask == "causal" else [8, 30, 5]
    x, q, k, v, do, bias = _case(lens, lkv, 2, 8, 13, mask, "softmax", bias_kind)
    dq, dk, dv, db = A.backward(q, k, v, x.q_off, x.kv_off, do, mask=mask, bias_kind=bias_kind, bias=bias)
    out, _ = A.forward(q, k, v, x.q_off, x.kv_off, mask=mask, bias_kind=bias_kind, bias=bias)
    for b in range(3):
        qs, qe, ks, ke = x.q_off[b], x.q_off[b + 1], x.kv_off[b], x.kv_off[b + 1]
        # adding one vector to every key shifts each row's scores by a constant
        np.testing.assert_allclose(dk[ks:ke].sum(axis=0), 0.0, atol=1e-12)
        # every row's probabilities sum to one
        np.testing.assert_allclose(dv[ks:ke].sum(axis=0), do[qs:qe].sum(axis=0), atol=1e-12)
        # scale Q by (1+t) and K by 1/(1+t): the scores do not move
        np.testing.assert_allclose((q[qs:qe] * dq[qs:qe]).sum(axis=(0, 2)),
                                   (k[ks:ke] * dk[ks:ke]).sum(axis=(0, 2)), atol=1e-12)
    if bias_kind == "scalar":
        np.testing.assert_allclose(db, 0.0, atol=1e-12)
    if bias_kind == "bucket":
        # a constant added to every table entry is a per-row shift: the table gradient sums to 0
        np.testing.assert_allclose(db.sum(axis=1), 0.0, atol=1e-12)
    # <dO, O> per row equals sum_j P dP; summed: <dO, O> = <dV, V>
    np.testing.assert_allclose((do * out).sum(), (dv * v).sum(), rtol=1e-12)


@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
def test_gdpa_invariants(act):
    lens = [7, 12]
    x, q, k, v, do, _ = _case(lens, lens, 2, 8, 14, "causal", act, "none")
    dq, dk, dv, _ = A.backward(q, k, v, x.q_off, x.kv_off, do, mask="causal", act=act)
    out, _ = A.forward(q, k, v, x.q_off, x.kv_off, mask="causal", act=act)
    # the output is linear in V
    np.testing.assert_allclose((dv * v).sum(), (do * out).sum(), rtol=1e-12)
    for b in range(2):
        s, e = x.q_off[b], x.q_off[b + 1]
        np.testing.assert_allclose((q[s:e] * dq[s:e]).sum(axis=(0, 2)), (k[s:e] * dk[s:e]).sum(axis=(0, 2)),
                                   atol=1e-12)


def test_empty_sequences_give_zero_gradients():
    x, q, k, v, do, _ = _case([3, 0, 2], [0, 4, 5], 2, 8, 15, "none", "softmax", "none")
    for act in ["softmax", "silu"]:
        dq, dk, dv, _ = A.backward(q, k, v, x.q_off, x.kv_off, do, act=act)
        np.testing.assert_array_equal(dq[:3], 0.0)
        np.testing.assert_array_equal(dk[:4], 0.0)
        np.testing.assert_array_equal(dv[:4], 0.0)
        assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk))


@pytest.mark.parametrize("mask,act,bias_kind", MODES)
@pytest.mark.parametrize("window", [0, 5])
def test_key_columns_match_library_autograd(mask, act, bias_kind, window):
    """oracle.key_cols evaluates dK_j and dV_j of single keys from their own score columns (the row
    statistics from whole rows); against torch autograd of padded dense attention, keys in any order."""
    lq, lkv = ([9, 17, 2, 30], [9, 17, 2, 30]) if mask == "causal" else ([9, 17, 2, 6], [12, 3, 20, 25])
    x, q, k, v, do, bias = _case(lq, lkv, 2, 16, 13, mask, act, bias_kind)
    scale = 1 / math.sqrt(16)
    if act == "softmax":
        _, _, _, rk, rv, _ = dense_softmax(q, k, v, x.q_off, x.kv_off, mask, bias_kind, bias, scale, want_grad=True,
                                           dout=do, window=window)
    else:
        _, _, rk, rv, _ = dense_gdpa(q, k, v, x.q_off, x.kv_off, mask, act, bias_kind, bias, scale, want_grad=True,
                                     dout=do, window=window)
    rng = np.random.default_rng(3)
    for b in range(4):
        L = lkv[b]
        keys = rng.permutation(L)[: max(1, L // 2)] if L else []
        for h in range(2):
            gk, gv = A.key_cols(q, k, v, x.q_off, x.kv_off, b, h, keys, do, mask=mask, act=act, bias_kind=bias_kind,
                                bias=bias, window=window)
            s = int(x.kv_off[b])
            np.testing.assert_allclose(gk, rk[s + np.asarray(keys, dtype=np.int64), h], rtol=0, atol=1e-11)
            np.testing.assert_allclose(gv, rv[s + np.asarray(keys, dtype=np.int64), h], rtol=0, atol=1e-11)


def test_key_columns_with_empty_rows_and_long_rows_in_chunks():
    """Rows that see no key contribute nothing; rows longer than one chunk give the same columns."""
    x, q, k, v, do, _ = _case([0, 3000], [5, 3000], 1, 8, 14, "none", "softmax", "none")
    keys = [0, 1, 2999, 1500]
    gk, gv = A.key_cols(q, k, v, x.q_off, x.kv_off, 1, 0, keys, do)
    _, dk, dv, _ = A.backward(q, k, v, x.q_off, x.kv_off, do, seqs=[1])
    np.testing.assert_allclose(gk, dk[5 + np.array(keys), 0], rtol=0, atol=1e-10)
    np.testing.assert_allclose(gv, dv[5 + np.array(keys), 0], rtol=0, atol=1e-10)
    gk0, gv0 = A.key_cols(q, k, v, x.q_off, x.kv_off, 0, 0, [0, 4], do)
    assert not gk0.any() and not gv0.any()
