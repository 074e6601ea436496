"""Pins of the oracle's window and block masks (CPU).

The oracle's visibility adds two limits to the base mask: a window (a query sees keys fewer than W
positions before it, and also after it without the causal mask) and a block size (query and key in
the same block of B positions). Pinned against torch's own attention kernels with the band as an
additive mask, against plain attention on sequences cut into blocks (a different path through
different offsets), against closed forms, and against finite differences.
"""
import math

import numpy as np
import pytest

import jfa_inputs as ji
from oracle import attention as A
from tests.oracle_pins_util import dense_gdpa, dense_softmax

f64 = A.bf16_bits_to_f64


def _case(lq, lkv, H, D, wid, mask, act, bias_kind):
    x = ji.make_inputs(lq, lkv, H, D, wid=wid, mask=mask, act=act, bias_kind=bias_kind, bias_sigma=0.5)
    bias = None if x.bias is None else x.bias.astype(np.float64)
    return x, f64(x.q), f64(x.k), f64(x.v), f64(x.do), bias


BANDS = [("causal", 5, 0), ("causal", 0, 8), ("causal", 6, 8), ("none", 4, 0), ("none", 0, 7), ("none", 3, 5)]


@pytest.mark.parametrize("mask,window,block", BANDS)
@pytest.mark.parametrize("bias_kind", ["none", "bucket"])
def test_softmax_band_matches_library_attention(mask, window, block, bias_kind):
    lens = [19, 1, 33, 8]
    x, q, k, v, do, bias = _case(lens, lens, 2, 16, 31, mask, "softmax", bias_kind)
    scale = 1 / math.sqrt(16)
    out, lse = A.forward(q, k, v, x.q_off, x.kv_off, mask=mask, bias_kind=bias_kind, bias=bias, window=window,
                         block=block)
    ref_out, ref_lse = dense_softmax(q, k, v, x.q_off, x.kv_off, mask, bias_kind, bias, scale, window=window,
                                     block=block)
    assert np.abs(out - ref_out).max() < 1e-12
    assert np.abs(lse - ref_lse).max() < 1e-12
    dq, dk, dv, db = A.backward(q, k, v, x.q_off, x.kv_off, do, mask=mask, bias_kind=bias_kind, bias=bias,
                                window=window, block=block)
    _, _, rq, rk, rv, rb = dense_softmax(q, k, v, x.q_off, x.kv_off, mask, bias_kind, bias, scale, want_grad=True,
                                         dout=do, window=window, block=block)
    for got, ref in [(dq, rq), (dk, rk), (dv, rv)] + ([(db, rb)] if rb is not None else []):
        assert np.abs(got - ref).max() < 1e-11


@pytest.mark.parametrize("mask,window,block", BANDS)
@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
def test_gdpa_band_matches_library_attention(mask, window, block, act):
    lens = [19, 1, 33, 8]
    x, q, k, v, do, bias = _case(lens, lens, 2, 16, 32, mask, act, "scalar")
    scale = 1 / math.sqrt(16)
    out, _ = A.forward(q, k, v, x.q_off, x.kv_off, mask=mask, act=act, bias_kind="scalar", bias=bias,
                       window=window, block=block)
    ref = dense_gdpa(q, k, v, x.q_off, x.kv_off, mask, act, "scalar", bias, scale, window=window, block=block)
    assert np.abs(out - ref[0]).max() < 1e-12
    dq, dk, dv, db = A.backward(q, k, v, x.q_off, x.kv_off, do, mask=mask, act=act, bias_kind="scalar", bias=bias,
                                window=window, block=block)
    g = dense_gdpa(q, k, v, x.q_off, x.kv_off, mask, act, "scalar", bias, scale, want_grad=True, dout=do,
                   window=window, block=block)
    for got, r in zip((dq, dk, dv, db), g[-4:]):
        assert np.abs(got - r).max() < 1e-11


@pytest.mark.parametrize("mask", ["causal", "none"])
def test_block_attention_is_attention_on_the_cut_sequences(mask):
    """Blocks of B positions attend only within themselves: the same as cutting every sequence into
    pieces of B and running plain attention on those (softmax, forward and backward)."""
    lens, B = [23, 5, 16, 1, 40], 8
    x, q, k, v, do, bias = _case(lens, lens, 2, 8, 33, mask, "softmax", "scalar")
    out, lse = A.forward(q, k, v, x.q_off, x.kv_off, mask=mask, bias_kind="scalar", bias=bias, block=B)
    grads = A.backward(q, k, v, x.q_off, x.kv_off, do, mask=mask, bias_kind="scalar", bias=bias, block=B)
    cut = []
    for L in lens:
        cut += [B] * (L // B) + ([L % B] if L % B else [])
    off = ji.offsets(cut)
    out2, lse2 = A.forward(q, k, v, off, off, mask=mask, bias_kind="scalar", bias=bias)
    grads2 = A.backward(q, k, v, off, off, do, mask=mask, bias_kind="scalar", bias=bias)
    assert np.abs(out - out2).max() < 1e-13
    assert np.abs(lse - lse2).max() < 1e-13
    for a, b in zip(grads[:3], grads2[:3]):
        assert np.abs(a - b).max() < 1e-13


def test_window_of_one_returns_each_rows_own_value():
    """Under the causal mask a window of 1 leaves each query only its own key: O_i = V_i exactly and
    lse_i = s_ii."""
    lens = [7, 1, 12]
    x, q, k, v, do, bias = _case(lens, lens, 3, 8, 34, "causal", "softmax", "bucket")
    out, lse = A.forward(q, k, v, x.q_off, x.kv_off, mask="causal", bias_kind="bucket", bias=bias, window=1)
    assert np.array_equal(out, v)
    s_ii = (q * k).sum(axis=2).T / math.sqrt(8) + bias[:, 0][:, None]  # bucket of distance 0
    assert np.abs(lse - s_ii).max() < 1e-12
    dq, dk, dv, db = A.backward(q, k, v, x.q_off, x.kv_off, do, mask="causal", bias_kind="bucket", bias=bias,
                                window=1)
    assert np.array_equal(dv, do) and np.all(dq == 0) and np.all(dk == 0) and np.all(db == 0)


@pytest.mark.parametrize("mask", ["causal", "none"])
def test_limits_longer_than_the_sequences_change_nothing(mask):
    lens = [9, 30, 2]
    x, q, k, v, do, bias = _case(lens, lens, 2, 8, 35, mask, "softmax", "bucket")
    base = A.forward(q, k, v, x.q_off, x.kv_off, mask=mask, bias_kind="bucket", bias=bias)
    band = A.forward(q, k, v, x.q_off, x.kv_off, mask=mask, bias_kind="bucket", bias=bias, window=30, block=30)
    assert np.array_equal(base[0], band[0]) and np.array_equal(base[1], band[1])


def _fd(fn, arr, h=1e-6):
    g = np.zeros_like(arr)
    flat, gf = arr.reshape(-1), g.reshape(-1)
    for n in range(flat.size):
        old = flat[n]
        flat[n] = old + h
        up = fn()
        flat[n] = old - h
        dn = fn()
        flat[n] = old
        gf[n] = (up - dn) / (2 * h)
    return g


@pytest.mark.parametrize("mask,act,window,block", [("causal", "softmax", 2, 0), ("none", "softmax", 0, 3),
                                                   ("causal", "silu", 2, 4), ("none", "gelu_tanh", 2, 0)])
def test_band_gradients_match_finite_differences(mask, act, window, block):
    lens = [5, 6, 1]
    x, q, k, v, do, bias = _case(lens, lens, 2, 4, 36, mask, act, "bucket")

    def loss():
        out, _ = A.forward(q, k, v, x.q_off, x.kv_off, mask=mask, act=act, bias_kind="bucket", bias=bias,
                           window=window, block=block)
        return float((out * do).sum())

    grads = A.backward(q, k, v, x.q_off, x.kv_off, do, mask=mask, act=act, bias_kind="bucket", bias=bias,
                       window=window, block=block)
    for got, arr in zip(grads, (q, k, v, bias)):
        ref = _fd(loss, arr)
        assert np.linalg.norm(got - ref) / max(1e-2, np.linalg.norm(ref)) < 1e-7


def test_bad_limits_are_rejected():
    x, q, k, v, do, bias = _case([3], [3], 1, 4, 37, "causal", "softmax", "none")
    for kw in [{"window": -1}, {"block": -2}, {"window": 1.5}]:
        with pytest.raises(ValueError):
            A.forward(q, k, v, x.q_off, x.kv_off, mask="causal", **kw)
