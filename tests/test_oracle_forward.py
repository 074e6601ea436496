"""Pins of the oracle's forward pass (CPU).

Each case compares the oracle with something other than itself: torch's CPU attention kernel on a
padded batch (brute force through a library routine), torch's activation routines, closed forms
and invariants.
"""
import math

import numpy as np
import pytest
import torch

import jfa_inputs as ji
from oracle import attention as A
from tests.oracle_pins_util import dense_gdpa, dense_softmax


def _case(lq, lkv, H, D, wid, mask, act, bias_kind, sigma=0.5):
    x = ji.make_inputs(lq, lkv, H, D, wid=wid, mask=mask, act=act, bias_kind=bias_kind, bias_sigma=sigma)
    f = A.bf16_bits_to_f64
    return x, f(x.q), f(x.k), f(x.v), f(x.do)


SHAPES = [
    ([5, 1, 9], [5, 1, 9]),
    ([7, 3], [7, 3]),
    ([1, 17, 4, 12], [1, 17, 4, 12]),
]
ASYM = [([3, 8, 1], [11, 2, 6]), ([4], [40])]


@pytest.mark.parametrize("bias_kind", ["none", "scalar", "bucket"])
@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("shape", range(len(SHAPES)))
def test_softmax_matches_library_attention(shape, mask, bias_kind):
    lq, lkv = SHAPES[shape]
    x, q, k, v, _ = _case(lq, lkv, 2, 8, 100 + shape, mask, "softmax", bias_kind)
    scale = 1 / math.sqrt(8)
    out, lse = A.forward(q, k, v, x.q_off, x.kv_off, mask=mask, bias_kind=bias_kind, bias=x.bias)
    ref_out, ref_lse = dense_softmax(q, k, v, x.q_off, x.kv_off, mask, bias_kind, x.bias, scale)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("bias_kind", ["none", "scalar", "bucket"])
@pytest.mark.parametrize("shape", range(len(ASYM)))
def test_softmax_asymmetric_lengths(shape, bias_kind):
    lq, lkv = ASYM[shape]
    x, q, k, v, _ = _case(lq, lkv, 3, 8, 200 + shape, "none", "softmax", bias_kind)
    out, lse = A.forward(q, k, v, x.q_off, x.kv_off, bias_kind=bias_kind, bias=x.bias)
    ref_out, ref_lse = dense_softmax(q, k, v, x.q_off, x.kv_off, "none", bias_kind, x.bias, 1 / math.sqrt(8))
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("bias_kind", ["none", "scalar", "bucket"])
def test_gdpa_matches_library_activations(act, mask, bias_kind):
    lq, lkv = ([6, 2, 13], [6, 2, 13]) if mask == "causal" else ([6, 2, 13], [9, 1, 4])
    x, q, k, v, _ = _case(lq, lkv, 2, 8, 300, mask, act, bias_kind)
    out, lse = A.forward(q, k, v, x.q_off, x.kv_off, mask=mask, act=act, bias_kind=bias_kind, bias=x.bias)
    assert lse is None
    (ref,) = dense_gdpa(q, k, v, x.q_off, x.kv_off, mask, act, bias_kind, x.bias, 1 / math.sqrt(8))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_activation_values():
    x = np.linspace(-12, 12, 2001)
    t = torch.from_numpy(x)
    np.testing.assert_allclose(A.silu(x), torch.nn.functional.silu(t).numpy(), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(A.gelu_tanh(x), torch.nn.functional.gelu(t, approximate="tanh").numpy(),
                               rtol=1e-14, atol=1e-15)
    # the tanh form stays within 1e-3 of the exact erf GELU everywhere
    assert np.max(np.abs(A.gelu_tanh(x) - torch.nn.functional.gelu(t).numpy())) < 1e-3
    assert A.silu(0.0) == 0.0 and A.gelu_tanh(0.0) == 0.0
    # derivatives against torch autograd of the library routines
    t.requires_grad_(True)
    for f, fp, tf in [(A.silu, A.silu_grad, lambda z: torch.nn.functional.silu(z)),
                      (A.gelu_tanh, A.gelu_tanh_grad, lambda z: torch.nn.functional.gelu(z, approximate="tanh"))]:
        (g,) = torch.autograd.grad(tf(t).sum(), t)
        np.testing.assert_allclose(fp(x), g.numpy(), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- closed forms and invariants

def _mk(lq, lkv, H=2, D=8, wid=7, **kw):
    return _case(lq, lkv, H, D, wid, kw.get("mask", "none"), kw.get("act", "softmax"), kw.get("bias_kind", "none"))


@pytest.mark.parametrize("mask", ["none", "causal"])
def test_constant_v_gives_constant_output(mask):
    x, q, k, v, _ = _mk([9, 4], [9, 4], mask=mask, bias_kind="bucket")
    v[:] = 0.0
    v[..., 3] = 2.5
    out, _ = A.forward(q, k, v, x.q_off, x.kv_off, mask=mask, bias_kind="bucket", bias=x.bias)
    expect = np.zeros_like(out)
    expect[..., 3] = 2.5
    np.testing.assert_allclose(out, expect, rtol=0, atol=1e-14)


def test_single_key_returns_that_value_row():
    x, q, k, v, _ = _mk([6, 3], [1, 1], bias_kind="scalar")
    out, _ = A.forward(q, k, v, x.q_off, x.kv_off, bias_kind="scalar", bias=x.bias)
    np.testing.assert_allclose(out[:6], np.broadcast_to(v[0], (6,) + v[0].shape), rtol=0, atol=0)
    np.testing.assert_allclose(out[6:], np.broadcast_to(v[1], (3,) + v[1].shape), rtol=0, atol=0)


def test_causal_first_row_is_first_value():
    x, q, k, v, _ = _mk([5, 7], [5, 7], mask="causal")
    out, lse = A.forward(q, k, v, x.q_off, x.kv_off, mask="causal")
    np.testing.assert_array_equal(out[0], v[0])
    np.testing.assert_array_equal(out[5], v[5])
    # row 0 sees one key: lse is its score
    s = (q[0] * k[0]).sum(-1) / math.sqrt(8)
    np.testing.assert_allclose(lse[:, 0], s, atol=1e-14)


@pytest.mark.parametrize("mask", ["none", "causal"])
def test_zero_queries_give_uniform_weights(mask):
    x, q, k, v, _ = _mk([6, 4], [6, 4], mask=mask)
    q[:] = 0.0
    out, lse = A.forward(q, k, v, x.q_off, x.kv_off, mask=mask)
    for b in range(2):
        s, e = x.q_off[b], x.q_off[b + 1]
        for i in range(e - s):
            n = (i + 1) if mask == "causal" else (e - s)
            np.testing.assert_allclose(out[s + i], v[s:s + n].mean(axis=0), atol=1e-14)
            np.testing.assert_allclose(lse[:, s + i], math.log(n), atol=1e-14)


def test_scalar_bias_shifts_lse_only():
    x, q, k, v, _ = _mk([5, 8], [7, 3], bias_kind="scalar")
    o0, l0 = A.forward(q, k, v, x.q_off, x.kv_off)
    o1, l1 = A.forward(q, k, v, x.q_off, x.kv_off, bias_kind="scalar", bias=x.bias)
    np.testing.assert_allclose(o1, o0, atol=1e-14)
    np.testing.assert_allclose(l1 - l0, np.broadcast_to(x.bias.astype(np.float64)[:, None], l0.shape), atol=1e-13)


def test_rows_of_p_sum_to_one_via_identity_values():
    # V_j = e_j (Lkv <= D): O_i is the probability row itself
    x, q, k, v, _ = _mk([5, 3], [6, 8], D=8, bias_kind="bucket")
    for b in range(2):
        s, e = x.kv_off[b], x.kv_off[b + 1]
        v[s:e] = 0.0
        for j in range(e - s):
            v[s + j, :, j] = 1.0
    out, _ = A.forward(q, k, v, x.q_off, x.kv_off, bias_kind="bucket", bias=x.bias)
    np.testing.assert_allclose(out.sum(axis=-1), 1.0, atol=1e-14)
    assert np.all(out >= 0)


def test_gdpa_closed_forms():
    x, q, k, v, _ = _mk([4, 6], [5, 2], act="silu")
    q[:] = 0.0
    for act in ["silu", "gelu_tanh"]:
        out, _ = A.forward(q, k, v, x.q_off, x.kv_off, act=act)
        np.testing.assert_array_equal(out, 0.0)
    c = np.array([0.7, -1.3])
    for act, f in [("silu", lambda z: z / (1 + math.exp(-z))),
                   ("gelu_tanh", lambda z: 0.5 * z * (1 + math.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3))))]:
        out, _ = A.forward(q, k, v, x.q_off, x.kv_off, act=act, bias_kind="scalar", bias=c)
        for b in range(2):
            qs, qe, ks, ke = x.q_off[b], x.q_off[b + 1], x.kv_off[b], x.kv_off[b + 1]
            for h in range(2):
                expect = f(c[h]) * v[ks:ke, h].sum(axis=0) / (ke - ks)
                np.testing.assert_allclose(out[qs:qe, h], np.broadcast_to(expect, (qe - qs, 8)), atol=1e-14)


def test_gdpa_linear_in_v():
    x, q, k, v, _ = _mk([5, 3], [4, 9], act="gelu_tanh", bias_kind="bucket")
    v2 = np.random.default_rng(3).standard_normal(v.shape)
    o1, _ = A.forward(q, k, v, x.q_off, x.kv_off, act="gelu_tanh", bias_kind="bucket", bias=x.bias)
    o2, _ = A.forward(q, k, v2, x.q_off, x.kv_off, act="gelu_tanh", bias_kind="bucket", bias=x.bias)
    o3, _ = A.forward(q, k, 2 * v - 3 * v2, x.q_off, x.kv_off, act="gelu_tanh", bias_kind="bucket", bias=x.bias)
    np.testing.assert_allclose(o3, 2 * o1 - 3 * o2, atol=1e-12)


def test_empty_sequences_and_rows():
    # a sequence with no keys: output 0, lse -inf; a sequence with no queries: nothing written
    x, q, k, v, _ = _mk([3, 0, 2], [0, 4, 5])
    out, lse = A.forward(q, k, v, x.q_off, x.kv_off)
    np.testing.assert_array_equal(out[:3], 0.0)
    assert np.all(np.isneginf(lse[:, :3]))
    assert np.all(np.isfinite(out[3:]))
    for act in ["silu", "gelu_tanh"]:
        out, _ = A.forward(q, k, v, x.q_off, x.kv_off, act=act)
        np.testing.assert_array_equal(out[:3], 0.0)


def test_packed_equals_concatenation_and_permutation():
    lens = [7, 2, 11, 5]
    x, q, k, v, _ = _mk(lens, lens, mask="causal", bias_kind="bucket")
    out, lse = A.forward(q, k, v, x.q_off, x.kv_off, mask="causal", bias_kind="bucket", bias=x.bias)
    off = x.q_off
    for b in range(4):
        s, e = off[b], off[b + 1]
        ob, lb = A.forward(q[s:e], k[s:e], v[s:e], [0, e - s], [0, e - s], mask="causal", bias_kind="bucket",
                           bias=x.bias)
        np.testing.assert_array_equal(ob, out[s:e])
        np.testing.assert_array_equal(lb, lse[:, s:e])
    perm = [2, 0, 3, 1]
    rows = np.concatenate([np.arange(off[b], off[b + 1]) for b in perm])
    poff = np.concatenate([[0], np.cumsum([lens[b] for b in perm])])
    op, lp = A.forward(q[rows], k[rows], v[rows], poff, poff, mask="causal", bias_kind="bucket", bias=x.bias)
    np.testing.assert_allclose(op, out[rows], atol=1e-15)
    np.testing.assert_allclose(lp, lse[:, rows], atol=1e-15)


def test_subset_selection_matches_full():
    x, q, k, v, _ = _mk([6, 9, 4], [6, 9, 4], H=3, mask="causal", bias_kind="bucket")
    full, lse = A.forward(q, k, v, x.q_off, x.kv_off, mask="causal", bias_kind="bucket", bias=x.bias)
    sub, lsub = A.forward(q, k, v, x.q_off, x.kv_off, mask="causal", bias_kind="bucket", bias=x.bias,
                          seqs=[1], heads=[0, 2])
    s, e = x.q_off[1], x.q_off[2]
    np.testing.assert_array_equal(sub[s:e][:, [0, 2]], full[s:e][:, [0, 2]])
    assert np.all(np.isnan(sub[:s])) and np.all(np.isnan(sub[s:e, 1]))


def test_gdpa_magnitude_bounds_output():
    x, q, k, v, _ = _mk([5, 9], [7, 4], act="silu", bias_kind="bucket")
    for act in ["silu", "gelu_tanh"]:
        out, _ = A.forward(q, k, v, x.q_off, x.kv_off, act=act, bias_kind="bucket", bias=x.bias)
        mag = A.gdpa_magnitude(q, k, v, x.q_off, x.kv_off, act=act, bias_kind="bucket", bias=x.bias)
        assert np.all(mag >= np.abs(out) - 1e-15)
    # every term non-negative: Q = 0 and a positive scalar bias give act(c) > 0; V >= 0
    q0 = np.zeros_like(q)
    va = np.abs(v)
    c = np.array([0.8, 1.5])
    out, _ = A.forward(q0, k, va, x.q_off, x.kv_off, act="gelu_tanh", bias_kind="scalar", bias=c)
    mag = A.gdpa_magnitude(q0, k, va, x.q_off, x.kv_off, act="gelu_tanh", bias_kind="scalar", bias=c)
    np.testing.assert_allclose(mag, out, rtol=1e-14)


@pytest.mark.parametrize("act", ["softmax", "silu", "gelu_tanh"])
@pytest.mark.parametrize("mask,window", [("causal", 0), ("none", 0), ("causal", 9)])
def test_row_by_row_equals_whole_batch(act, mask, window):
    """oracle.rows (one score row at a time) reproduces forward / backward on the same rows."""
    import jfa_inputs as ji
    lens = [30, 1, 45]
    x = ji.make_inputs(lens, lens, 2, 8, wid=61, mask=mask, act=act, bias_kind="bucket", bias_sigma=0.7,
                       window=window)
    f = A.bf16_bits_to_f64
    q, k, v, do = f(x.q), f(x.k), f(x.v), f(x.do)
    kw = dict(mask=mask, act=act, bias_kind="bucket", bias=x.bias.astype(np.float64), window=window)
    out, lse = A.forward(q, k, v, x.q_off, x.kv_off, **kw)
    dq, _, _, _ = A.backward(q, k, v, x.q_off, x.kv_off, do, **kw)
    for b, h, sel in [(0, 1, [0, 7, 29]), (2, 0, [44, 3]), (1, 1, [0])]:
        o, l, g = A.rows(q, k, v, x.q_off, x.kv_off, b, h, sel, do, **kw)
        idx = [x.q_off[b] + i for i in sel]
        np.testing.assert_allclose(o, out[idx, h], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g, dq[idx, h], rtol=1e-10, atol=1e-12)
        if act == "softmax":
            np.testing.assert_allclose(l, lse[h, idx], rtol=1e-12, atol=1e-12)
