"""The oracle's pins catch plausible mistakes (CPU).

Each case plants one mistake in a private copy of the oracle's source (a dropped term, a wrong
index or sign, a wrong normaliser), loads that copy as a separate module and requires that the
library-based pins reject it. The real oracle is never modified.
"""
import math
import os
import types

import numpy as np
import pytest

import jfa_inputs as ji
from oracle import attention as A
from tests.oracle_pins_util import dense_gdpa, dense_softmax

_SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")
with open(_SRC_PATH) as f:
    _SRC = f.read()


def _mutant(old, new):
    assert _SRC.count(old) >= 1, old
    mod = types.ModuleType("oracle._attention_mutant")
    mod.__package__ = "oracle"
    exec(compile(_SRC.replace(old, new, 1), "mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod):
    """True when the mutated oracle passes forward and backward library pins on small cases."""
    D = 8
    scale = 1 / math.sqrt(D)
    for mask, act, bias_kind in [("causal", "softmax", "bucket"), ("none", "softmax", "scalar"),
                                 ("causal", "silu", "bucket"), ("none", "gelu_tanh", "scalar"),
                                 ("causal", "gelu_tanh", "none")]:
        lq = [5, 19, 2]
        lkv = lq if mask == "causal" else [7, 3, 22]
        x = ji.make_inputs(lq, lkv, 2, D, wid=21, mask=mask, act=act, bias_kind=bias_kind, bias_sigma=0.5)
        f = A.bf16_bits_to_f64
        q, k, v, do = f(x.q), f(x.k), f(x.v), f(x.do)
        bias = None if x.bias is None else x.bias.astype(np.float64)
        try:
            out, lse = mod.forward(q, k, v, x.q_off, x.kv_off, mask=mask, act=act, bias_kind=bias_kind, bias=bias)
            grads = mod.backward(q, k, v, x.q_off, x.kv_off, do, mask=mask, act=act, bias_kind=bias_kind,
                                 bias=bias)
        except Exception:
            return False
        if act == "softmax":
            r_out, r_lse = dense_softmax(q, k, v, x.q_off, x.kv_off, mask, bias_kind, bias, scale)
            _, _, *rg = dense_softmax(q, k, v, x.q_off, x.kv_off, mask, bias_kind, bias, scale, True, do)
            if not np.allclose(lse, r_lse, rtol=0, atol=1e-10):
                return False
        else:
            (r_out,) = dense_gdpa(q, k, v, x.q_off, x.kv_off, mask, act, bias_kind, bias, scale)
            _, *rg = dense_gdpa(q, k, v, x.q_off, x.kv_off, mask, act, bias_kind, bias, scale, True, do)
        if not np.allclose(out, r_out, rtol=0, atol=1e-10):
            return False
        for g, r in zip(grads, rg):
            if (g is None) != (r is None) or (g is not None and not np.allclose(g, r, rtol=0, atol=1e-10)):
                return False
    return True


MUTATIONS = [
    ("causal mask off by one", "vis = (j <= i) if mask", "vis = (j < i) if mask"),
    ("scale dropped", "S = scale * (Qc @ K.T)", "S = (Qc @ K.T)"),
    ("scale applied after the bias", "S = S + bias_h[bucket(i - j)]", "S = S + scale * bias_h[bucket(i - j)]"),
    ("bucket index shifted", "S = S + bias_h[bucket(i - j)]", "S = S + bias_h[bucket(i - j + 1)]"),
    ("bucket of j - i with sign kept", "S = S + bias_h[bucket(i - j)]", "S = S + bias_h[np.minimum(63, np.maximum(0, j - i))]"),
    ("lse without the log-sum", "lse = np.where(any_vis, m + np.log(np.where(any_vis, l, 1.0)), -np.inf)",
     "lse = np.where(any_vis, m, -np.inf)"),
    ("GDPA normaliser dropped", "out[qs + i0:qs + i1, h] = (A @ V) / lkv if lkv > 0 else 0.0",
     "out[qs + i0:qs + i1, h] = (A @ V) if lkv > 0 else 0.0"),
    ("GDPA masked entries not zeroed", "A = np.where(vis, f(S), 0.0)\n                    out",
     "A = f(S)\n                    out"),
    ("softmax Delta term dropped", "dS = P * (dP - delta[:, None])", "dS = P * dP"),
    ("dS sign flipped", "dS = P * (dP - delta[:, None])", "dS = P * (delta[:, None] - dP)"),
    ("dK without scale", "dK += scale * (dS.T @ Qc)", "dK += dS.T @ Qc"),
    ("dQ from V instead of K", "dq[qs + i0:qs + i1, h] = scale * (dS @ K)", "dq[qs + i0:qs + i1, h] = scale * (dS @ V)"),
    ("GDPA dV normaliser dropped", "dV += (A.T @ dOc) * inv_l", "dV += A.T @ dOc"),
    ("SiLU derivative wrong", "return sig * (1.0 + x * (1.0 - sig))", "return sig * (1.0 + x * sig)"),
    ("GELU derivative term dropped", "return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * du",
     "return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t) * du"),
    ("GELU cubic coefficient wrong", "_GELU_C = 0.044715", "_GELU_C = 0.0447"),
    ("bucket bias gradient to the wrong bucket", "weights=dS[vis], minlength", "weights=dS.T[vis.T], minlength"),
]


def test_real_oracle_passes():
    assert _pins_pass(A)


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    assert not _pins_pass(_mutant(old, new)), name


def _band_pins_pass(mod):
    """True when the mutated oracle passes library pins with window and block limits."""
    D = 8
    scale = 1 / math.sqrt(D)
    lens = [13, 2, 21]
    for mask, act, window, block in [("causal", "softmax", 4, 0), ("none", "softmax", 3, 0), ("causal", "softmax", 0, 5),
                                     ("none", "silu", 0, 6), ("causal", "gelu_tanh", 3, 8)]:
        x = ji.make_inputs(lens, lens, 2, D, wid=22, mask=mask, act=act, bias_kind="bucket", bias_sigma=0.5)
        f = A.bf16_bits_to_f64
        q, k, v, do = f(x.q), f(x.k), f(x.v), f(x.do)
        bias = x.bias.astype(np.float64)
        kw = dict(mask=mask, act=act, bias_kind="bucket", bias=bias, window=window, block=block)
        try:
            out, _ = mod.forward(q, k, v, x.q_off, x.kv_off, **kw)
            grads = mod.backward(q, k, v, x.q_off, x.kv_off, do, **kw)
        except Exception:
            return False
        if act == "softmax":
            r_out, _ = dense_softmax(q, k, v, x.q_off, x.kv_off, mask, "bucket", bias, scale, window=window, block=block)
            _, _, *rg = dense_softmax(q, k, v, x.q_off, x.kv_off, mask, "bucket", bias, scale, True, do,
                                      window=window, block=block)
        else:
            (r_out,) = dense_gdpa(q, k, v, x.q_off, x.kv_off, mask, act, "bucket", bias, scale, window=window,
                                  block=block)
            _, *rg = dense_gdpa(q, k, v, x.q_off, x.kv_off, mask, act, "bucket", bias, scale, True, do,
                                window=window, block=block)
        if not np.allclose(out, r_out, rtol=0, atol=1e-10):
            return False
        for g, r in zip(grads, rg):
            if not np.allclose(g, r, rtol=0, atol=1e-10):
                return False
    return True


BAND_MUTATIONS = [
    ("window off by one", "vis = vis & (i - j < window)", "vis = vis & (i - j <= window)"),
    ("window without its forward side", "vis = vis & (j - i < window)", "vis = vis & (j - i < 10 ** 9)"),
    ("block boundary shifted", "vis = vis & (i // block == j // block)", "vis = vis & ((i + 1) // block == j // block)"),
    ("block ignored", "vis = vis & (i // block == j // block)", "vis = vis"),
]


def test_real_oracle_passes_band_pins():
    assert _band_pins_pass(A)


@pytest.mark.parametrize("name,old,new", BAND_MUTATIONS, ids=[m[0] for m in BAND_MUTATIONS])
def test_planted_band_mistake_is_caught(name, old, new):
    assert not _band_pins_pass(_mutant(old, new)), name


def _keycols_pins_pass(mod):
    """True when the mutated oracle's per-key gradients pass library autograd pins."""
    D = 8
    scale = 1 / math.sqrt(D)
    for mask, act, bias_kind in [("causal", "softmax", "bucket"), ("none", "softmax", "scalar"),
                                 ("causal", "silu", "bucket"), ("none", "gelu_tanh", "none")]:
        lq = [5, 19, 2]
        lkv = lq if mask == "causal" else [7, 3, 22]
        x = ji.make_inputs(lq, lkv, 2, D, wid=23, mask=mask, act=act, bias_kind=bias_kind, bias_sigma=0.5)
        f = A.bf16_bits_to_f64
        q, k, v, do = f(x.q), f(x.k), f(x.v), f(x.do)
        bias = None if x.bias is None else x.bias.astype(np.float64)
        if act == "softmax":
            _, _, _, rk, rv, _ = dense_softmax(q, k, v, x.q_off, x.kv_off, mask, bias_kind, bias, scale, True, do)
        else:
            _, _, rk, rv, _ = dense_gdpa(q, k, v, x.q_off, x.kv_off, mask, act, bias_kind, bias, scale, True, do)
        for b in range(3):
            keys = np.arange(lkv[b])[::-2]  # a subset of the keys, in reverse order
            s = int(x.kv_off[b])
            for h in range(2):
                try:
                    gk, gv = mod.key_cols(q, k, v, x.q_off, x.kv_off, b, h, keys, do, mask=mask, act=act,
                                          bias_kind=bias_kind, bias=bias)
                except Exception:
                    return False
                if not (np.allclose(gk, rk[s + keys, h], rtol=0, atol=1e-10)
                        and np.allclose(gv, rv[s + keys, h], rtol=0, atol=1e-10)):
                    return False
    return True


KEYCOL_MUTATIONS = [
    ("Delta from the selected columns only", "delta = (P * (dOc @ V.T)).sum(axis=1)",
     "delta = (P[:, keys] * (dOc @ V[keys].T)).sum(axis=1)"),
    ("bias at the column index instead of the key position", "Sk = Sk + bias_h[bucket(i - j)]",
     "Sk = Sk + bias_h[bucket(i - np.arange(len(keys))[None, :])]"),
    ("probabilities without the row's lse", "np.exp(Sk - np.where(np.isfinite(lse), lse, 0.0)[:, None])",
     "np.exp(Sk)"),
    ("visibility of the column index", "visk = visible(i, j, mask, window, block) & (j < lkv)",
     "visk = visible(i, np.arange(len(keys))[None, :], mask, window, block) & (j < lkv)"),
    ("per-key dK without scale", "dk += scale * (dSk.T @ Qc)", "dk += dSk.T @ Qc"),
    ("per-key dV from Q", "dv += Pk.T @ dOc", "dv += Pk.T @ Qc"),
    ("GDPA per-key normaliser dropped", "Pk = np.where(visk, f(Sk), 0.0) * inv_l", "Pk = np.where(visk, f(Sk), 0.0)"),
]


def test_real_oracle_passes_key_column_pins():
    assert _keycols_pins_pass(A)


@pytest.mark.parametrize("name,old,new", KEYCOL_MUTATIONS, ids=[m[0] for m in KEYCOL_MUTATIONS])
def test_planted_key_column_mistake_is_caught(name, old, new):
    assert not _keycols_pins_pass(_mutant(old, new)), name
