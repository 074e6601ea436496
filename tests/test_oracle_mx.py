"""Pins of the MXFP8 oracle (CPU): the E4M3 rounding against torch's float8_e4m3fn conversion and a
brute-force search over every E4M3 code, the block scale against torch.frexp, closed forms of the
MXFP8 attention forward, and an independent torch implementation of it that quantises with torch's
own float8 conversion."""
import math

import numpy as np
import pytest
import torch

import jfa_inputs as ji
from oracle import attention as A
from oracle import mx

f = A.bf16_bits_to_f64


def _codes():
    """Every finite E4M3 value with its code (sign, 4 exponent bits, bias 7, 3 mantissa bits)."""
    vals = []
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue  # NaN
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        v = math.ldexp(1 + m / 8, e - 7) if e else math.ldexp(m / 8, -6)
        vals.append((-v if s else v, c))
    return vals


def _brute(x):
    best = None
    for v, c in _codes():
        d = abs(v - x)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0 and (best[1] & 1) == 1):
            best = (d, c, v)
    return best[2]


def test_e4m3_rounding_matches_torch_and_brute_force():
    rng = np.random.default_rng(0)
    vals = sorted(v for v, _ in _codes())
    mids = [(a + b) / 2 for a, b in zip(vals[:-1], vals[1:])]
    x = np.concatenate([rng.uniform(-448, 448, 2000), np.exp2(rng.uniform(-12, 8.8, 2000)) * rng.choice([-1, 1], 2000),
                        np.array(mids), np.array(vals)])
    got = mx.e4m3_round(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, ref)
    for xi in np.concatenate([x[::97], np.array(mids[::5])]):
        assert mx.e4m3_round(xi) == _brute(xi), xi
    # saturation above the largest value
    np.testing.assert_array_equal(mx.e4m3_round(np.array([449.0, 470.0, 511.0, -1e6])), [448, 448, 448, -448])


def test_block_scale_and_quantize():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 96)) * np.exp2(rng.integers(-20, 20, (7, 1)))
    x[3, 32:64] = 0.0  # an all-zero block
    q = mx.mx_quantize(x, axis=1)
    b = torch.from_numpy(x.reshape(7, 3, 32))
    amax = b.abs().amax(-1)
    _, ex = torch.frexp(amax)  # amax = m 2^ex, 0.5 <= m < 1
    scale = torch.where(amax > 0, torch.exp2((ex - 1 - 8).double()), torch.tensor(2.0 ** -127, dtype=torch.float64))
    ref = ((b / scale[..., None]).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64) * scale[..., None])
    np.testing.assert_array_equal(q, ref.reshape(7, 96).numpy())
    assert not q[3, 32:64].any()
    np.testing.assert_array_equal(mx.mx_quantize(q, axis=1), q)                  # idempotent
    np.testing.assert_array_equal(mx.mx_quantize(x * 2.0 ** 5, axis=1), q * 2.0 ** 5)  # power-of-two equivariant
    # every element within 2^-3 of its block's largest magnitude (half a quantum of the top binade is
    # 2^-4 of it; saturation of x / scale in (448, 512) to 448 costs at most 64 / 512)
    err = np.abs(q - x).reshape(7, 3, 32)
    amax = np.abs(x).reshape(7, 3, 32).max(-1, keepdims=True)
    assert np.all(err <= amax * 2.0 ** -3)
    sat = np.abs(x).reshape(7, 3, 32) / mx.mx_block_scale(amax) > 448
    assert np.all(err[~sat] <= (amax * 2.0 ** -4).repeat(32, -1)[~sat])


def _torch_mx_forward(q, k, v, q_off, kv_off, mask, bias_kind, bias, scale):
    """The MXFP8 forward with every quantisation done by torch's float8_e4m3fn conversion."""
    def quant(t, dim):
        t = t.movedim(dim, -1)
        n = t.shape[-1]
        pad = (-n) % 32
        tp = torch.nn.functional.pad(t, (0, pad)).reshape(*t.shape[:-1], -1, 32)
        amax = tp.abs().amax(-1, keepdim=True)
        _, ex = torch.frexp(amax)
        sc = torch.where(amax > 0, torch.exp2((ex - 9).double()), torch.tensor(2.0 ** -127, dtype=torch.float64))
        r = (tp / sc).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64) * sc
        return r.reshape(*t.shape[:-1], -1)[..., :n].movedim(-1, dim)

    from tests.oracle_pins_util import dense_bias_and_mask, padded, unpad
    H, D = q.shape[1], q.shape[2]
    Lq, Lk = int(np.diff(q_off).max()), int(np.diff(kv_off).max())
    Q = quant(padded(q, q_off, Lq), -1)
    K = quant(padded(k, kv_off, Lk), -1)
    V = quant(padded(v, kv_off, Lk), 2)  # along keys from each sequence's first key
    add, vis = dense_bias_and_mask(q_off, kv_off, H, Lq, Lk, mask, bias_kind, bias)
    x = (scale * Q @ K.transpose(-1, -2) + add) / math.log(2.0)
    x = torch.where(vis, x, torch.tensor(-math.inf, dtype=x.dtype))
    M = torch.ceil(torch.nan_to_num(x.amax(-1, keepdim=True), neginf=0.0))
    Pt = torch.where(vis, torch.exp2(x - M), torch.zeros_like(x))
    Pq = quant(Pt, -1)
    l = Pt.sum(-1, keepdim=True)
    out = torch.where(l > 0, (Pq @ V) / torch.where(l > 0, l, torch.ones_like(l)), torch.zeros_like(l))
    return unpad(out, q_off)


@pytest.mark.parametrize("mask,bias_kind", [("none", "none"), ("causal", "bucket"), ("none", "scalar")])
def test_mx_forward_matches_an_implementation_on_torch_float8(mask, bias_kind):
    lq = [7, 40, 1, 70]
    lkv = lq if mask == "causal" else [33, 5, 64, 100]
    x = ji.make_inputs(lq, lkv, 2, 64, wid=90, mask=mask, act="softmax", bias_kind=bias_kind, bias_sigma=0.5)
    q, k, v = f(x.q), f(x.k), f(x.v)
    bias = None if x.bias is None else x.bias.astype(np.float64)
    out, lse = mx.forward(q, k, v, x.q_off, x.kv_off, mask=mask, bias_kind=bias_kind, bias=bias)
    ref = _torch_mx_forward(q, k, v, x.q_off, x.kv_off, mask, bias_kind, bias, 1 / 8)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # lse is the exact log-sum-exp of the scores from the quantised Q and K
    qh, kh = mx.mx_quantize(q), mx.mx_quantize(k)
    _, l2 = A.forward(qh, kh, v, x.q_off, x.kv_off, mask=mask, bias_kind=bias_kind, bias=bias)
    np.testing.assert_allclose(lse, l2, rtol=0, atol=1e-12)


def test_mx_forward_closed_forms():
    lens = [5, 64, 100]
    x = ji.make_inputs(lens, lens, 2, 64, wid=91, mask="causal")
    v = f(x.v)
    z = np.zeros_like(f(x.q))
    out, lse = mx.forward(z, f(x.k), v, x.q_off, x.kv_off, mask="causal")
    # Q = 0: every visible score is 0, P~ = 1 exactly; out_i is the prefix mean of the quantised values
    for b, L in enumerate(lens):
        s = int(x.kv_off[b])
        vh = mx._quantize_seq_keys(v[s:s + L, 0])
        np.testing.assert_allclose(out[s:s + L, 0], np.cumsum(vh, 0) / np.arange(1, L + 1)[:, None], rtol=1e-13)
        np.testing.assert_allclose(lse[0, s:s + L], np.log(np.arange(1, L + 1)), rtol=0, atol=1e-13)
    # a power of two on V scales the output by the same power exactly
    q, k = f(x.q), f(x.k)
    o1, _ = mx.forward(q, k, v, x.q_off, x.kv_off, mask="causal")
    o2, _ = mx.forward(q, k, v * 8.0, x.q_off, x.kv_off, mask="causal")
    np.testing.assert_array_equal(o2, o1 * 8.0)


def test_mx_forward_is_close_to_the_full_precision_result():
    """The quantisation error of the MXFP8 forward on N(0,1) inputs against
    the full-precision oracle: 5.9% on this case (the GPU numerics gate, rel-L2 <= 0.1, keeps a margin)."""
    lens = [300, 64, 1000]
    x = ji.make_inputs(lens, lens, 2, 128, wid=92, mask="causal", bias_kind="bucket", bias_sigma=0.5)
    q, k, v = f(x.q), f(x.k), f(x.v)
    kw = dict(mask="causal", bias_kind="bucket", bias=x.bias.astype(np.float64))
    o_mx, l_mx = mx.forward(q, k, v, x.q_off, x.kv_off, **kw)
    o, l = A.forward(q, k, v, x.q_off, x.kv_off, **kw)
    rel = np.linalg.norm(o_mx - o) / np.linalg.norm(o)
    assert 1e-2 < rel < 0.1, rel  # 5.9% here
    assert np.abs(l_mx - l).max() < 0.15  # 0.064 here
