"""Pins of the oracle for shared queries (pooling by multihead attention) and for the fused
self + target pass (causal with more queries than keys), on the CPU.

Shared queries: against torch's attention on a padded batch whose query tensor is the seed tensor
expanded over the batch (torch's own broadcast; its backward sums the seed gradient over the batch).
Fused pass: against torch on a padded batch with the explicit mask, and against two separate oracle
calls (causal self-attention of the history, then attention of the targets on the history).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import jfa_inputs as ji
from oracle import attention as A
from tests.oracle_pins_util import dense_gdpa, dense_softmax, padded, unpad

f = A.bf16_bits_to_f64


def _seed_case(Ls, lkv, H, D, act, bias_kind, wid=31):
    x = ji.make_inputs([Ls] * len(lkv), lkv, H, D, wid=wid, mask="none", act=act, bias_kind=bias_kind, bias_sigma=0.5)
    seeds = f(x.q[:Ls])  # the first sequence's rows serve as the shared seeds
    bias = None if x.bias is None else x.bias.astype(np.float64)
    return x, seeds, f(x.k), f(x.v), f(x.do), bias


@pytest.mark.parametrize("act", ["softmax", "silu", "gelu_tanh"])
@pytest.mark.parametrize("bias_kind", ["none", "scalar", "bucket"])
def test_shared_queries_match_library_broadcast(act, bias_kind):
    Ls, lkv, H, D = 5, [7, 1, 19, 2, 4], 2, 8
    x, seeds, k, v, do, bias = _seed_case(Ls, lkv, H, D, act, bias_kind)
    scale = 1 / math.sqrt(D)
    kw = dict(act=act, bias_kind=bias_kind, bias=bias)
    out, lse = A.forward_shared_q(seeds, k, v, x.kv_off, **kw)
    dq, dk, dv, db = A.backward_shared_q(seeds, k, v, x.kv_off, do, **kw)
    assert dq.shape == seeds.shape
    # torch: seeds as a leaf, broadcast by expand (no copy); autograd sums over the batch
    B = len(lkv)
    S = torch.from_numpy(seeds.transpose(1, 0, 2).copy()).requires_grad_(True)  # [H, Ls, D]
    q_off = np.arange(B + 1) * Ls
    q_rep = np.tile(seeds, (B, 1, 1))
    if act == "softmax":
        r = dense_softmax(q_rep, k, v, q_off, x.kv_off, "none", bias_kind, bias, scale, True, do)
        r_out, r_dk, r_dv = r[0], r[3], r[4]
    else:
        r = dense_gdpa(q_rep, k, v, q_off, x.kv_off, "none", act, bias_kind, bias, scale, True, do)
        r_out, r_dk, r_dv = r[0], r[2], r[3]
    np.testing.assert_allclose(out, r_out, rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, r_dk, rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, r_dv, rtol=0, atol=1e-11)
    # the seed gradient through torch's own broadcast: padded keys per sequence, softmax or GDPA
    Lk = max(lkv)
    K, V = padded(k, x.kv_off, Lk), padded(v, x.kv_off, Lk)
    Q = S[None].expand(B, H, Ls, D)
    s = scale * (Q @ K.transpose(-1, -2))
    j = torch.arange(Lk)[None, None, None, :]
    lk = torch.tensor(lkv)[:, None, None, None]
    if bias_kind == "scalar":
        s = s + torch.from_numpy(bias)[None, :, None, None]
    elif bias_kind == "bucket":
        from tests.oracle_pins_util import bucket_by_boundaries
        idx = torch.from_numpy(bucket_by_boundaries(np.arange(Ls)[:, None] - np.arange(Lk)[None, :]))
        s = s + torch.from_numpy(bias)[:, idx][None]
    vis = j < lk
    if act == "softmax":
        p = torch.softmax(torch.where(vis, s, torch.tensor(-math.inf, dtype=s.dtype)), dim=-1)
        p = torch.nan_to_num(p, nan=0.0)  # a sequence with no key: zero weights
    else:
        fn = F.silu if act == "silu" else (lambda t: F.gelu(t, approximate="tanh"))
        p = torch.where(vis, fn(s), torch.zeros_like(s)) / torch.clamp(lk, min=1)
    o = p @ V
    dO = padded(do, q_off, Ls)
    (o * dO).sum().backward()
    np.testing.assert_allclose(dq, S.grad.numpy().transpose(1, 0, 2), rtol=0, atol=1e-11)


def test_shared_queries_equal_explicit_replication():
    Ls, lkv, H, D = 3, [4, 9, 2], 2, 8
    x, seeds, k, v, do, bias = _seed_case(Ls, lkv, H, D, "softmax", "bucket")
    q_rep, q_off = A.replicate_shared_q(seeds, 3)
    assert q_rep.shape == (9, H, D) and list(q_off) == [0, 3, 6, 9]
    for b in range(3):
        np.testing.assert_array_equal(q_rep[3 * b:3 * b + 3], seeds)
    o1, l1 = A.forward_shared_q(seeds, k, v, x.kv_off, bias_kind="bucket", bias=bias)
    o2, l2 = A.forward(q_rep, k, v, q_off, x.kv_off, bias_kind="bucket", bias=bias)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    dq, *_ = A.backward_shared_q(seeds, k, v, x.kv_off, do, bias_kind="bucket", bias=bias)
    dq_rep, *_ = A.backward(q_rep, k, v, q_off, x.kv_off, do, bias_kind="bucket", bias=bias)
    np.testing.assert_allclose(dq, dq_rep[0:3] + dq_rep[3:6] + dq_rep[6:9], rtol=0, atol=1e-14)
    # a sequence with no key: zero output and no contribution to the seed gradient
    x0, s0, k0, v0, do0, _ = _seed_case(Ls, [4, 0], H, D, "softmax", "none")
    o0, l0 = A.forward_shared_q(s0, k0, v0, x0.kv_off)
    assert not o0[3:].any() and np.all(l0[:, 3:] == -np.inf)
    g0 = A.backward_shared_q(s0, k0, v0, x0.kv_off, do0)[0]
    g1 = A.backward(s0, k0[:4], v0[:4], np.array([0, 3]), np.array([0, 4]), do0[:3])[0]
    np.testing.assert_allclose(g0, g1, rtol=0, atol=1e-14)


MODES = [(a, b) for a in ("softmax", "silu", "gelu_tanh") for b in ("none", "scalar", "bucket")]


@pytest.mark.parametrize("act,bias_kind", MODES)
def test_self_plus_target_matches_library_mask(act, bias_kind):
    """Causal with Lq > Lkv: history rows causal, target rows see the whole history."""
    lh, lc = [6, 1, 13, 3], [4, 2, 0, 7]
    lq = [a + b for a, b in zip(lh, lc)]
    x = ji.make_inputs(lq, lh, 2, 8, wid=32, mask="causal", act=act, bias_kind=bias_kind, bias_sigma=0.5)
    q, k, v, do = f(x.q), f(x.k), f(x.v), f(x.do)
    bias = None if x.bias is None else x.bias.astype(np.float64)
    scale = 1 / math.sqrt(8)
    kw = dict(mask="causal", act=act, bias_kind=bias_kind, bias=bias)
    out, lse = A.forward(q, k, v, x.q_off, x.kv_off, **kw)
    grads = A.backward(q, k, v, x.q_off, x.kv_off, do, **kw)
    if act == "softmax":
        r = dense_softmax(q, k, v, x.q_off, x.kv_off, "causal", bias_kind, bias, scale, True, do)
        r_out, r_grads = r[0], r[2:]
        r_lse = dense_softmax(q, k, v, x.q_off, x.kv_off, "causal", bias_kind, bias, scale)[1]
        np.testing.assert_allclose(lse, r_lse, rtol=0, atol=1e-11)
    else:
        r = dense_gdpa(q, k, v, x.q_off, x.kv_off, "causal", act, bias_kind, bias, scale, True, do)
        r_out, r_grads = r[0], r[1:]
    np.testing.assert_allclose(out, r_out, rtol=0, atol=1e-11)
    for g, rg in zip(grads, r_grads):
        if g is None:
            assert rg is None
        else:
            np.testing.assert_allclose(g, rg, rtol=0, atol=1e-11)


@pytest.mark.parametrize("act", ["softmax", "silu"])
@pytest.mark.parametrize("bias_kind", ["none", "scalar"])
def test_self_plus_target_equals_two_separate_calls(act, bias_kind):
    """The fused pass gives the causal self-attention of the history on history rows and the
    unmasked attention of the targets on the history on target rows; key gradients add up."""
    lh, lc = [6, 1, 13, 3], [4, 2, 0, 7]
    lq = [a + b for a, b in zip(lh, lc)]
    x = ji.make_inputs(lq, lh, 2, 8, wid=33, mask="causal", act=act, bias_kind=bias_kind, bias_sigma=0.5)
    q, k, v, do = f(x.q), f(x.k), f(x.v), f(x.do)
    bias = None if x.bias is None else x.bias.astype(np.float64)
    kw = dict(act=act, bias_kind=bias_kind, bias=bias)
    out, lse = A.forward(q, k, v, x.q_off, x.kv_off, mask="causal", **kw)
    dq, dk, dv, db = A.backward(q, k, v, x.q_off, x.kv_off, do, mask="causal", **kw)
    hist = np.concatenate([np.arange(x.q_off[b], x.q_off[b] + lh[b]) for b in range(4)])
    targ = np.concatenate([np.arange(x.q_off[b] + lh[b], x.q_off[b + 1]) for b in range(4)])
    off_h, off_t = ji.offsets(lh), ji.offsets(lc)
    o1, l1 = A.forward(q[hist], k, v, off_h, x.kv_off, mask="causal", **kw)
    o2, l2 = A.forward(q[targ], k, v, off_t, x.kv_off, mask="none", **kw)
    np.testing.assert_allclose(out[hist], o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(out[targ], o2, rtol=0, atol=1e-13)
    g1 = A.backward(q[hist], k, v, off_h, x.kv_off, do[hist], mask="causal", **kw)
    g2 = A.backward(q[targ], k, v, off_t, x.kv_off, do[targ], mask="none", **kw)
    np.testing.assert_allclose(dq[hist], g1[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dq[targ], g2[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk, g1[1] + g2[1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, g1[2] + g2[2], rtol=0, atol=1e-12)
