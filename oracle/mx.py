"""MXFP8 attention forward, written from its definition (test infrastructure only).

The pages train attention in MXFP8 with block quantisation and convert the probabilities P to MXFP8
online (kerneldigest.dev page, "Arquitectura del Sistema"). MXFP8 is the microscaling format: a
block of 32 elements shares one power-of-two scale (an 8-bit exponent, E8M0) and each element is
an FP8 E4M3 number (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest value 448, no
infinities). The pages fix neither the block rule nor the blocks, so these are readings:

  * scale of a block: 2^(floor(log2 amax) - 8), amax the block's largest magnitude (8 is the
    exponent of E4M3's largest power of two, 256); an all-zero block has scale 2^-127;
  * element: x / scale rounded to the nearest E4M3 value, ties to even mantissa, magnitudes above
    448 saturating to 448;
  * Q and K: blocks of 32 consecutive features of a row (four per row at D = 128);
  * V: blocks of 32 consecutive keys of one feature, counted from the sequence's first key (the
    last block of a sequence is padded with zeros);
  * scores from the dequantised Q and K in full precision: s_ij = scale <Q^_i, K^_j> + bias;
  * probabilities: with x_ij = s_ij log2(e) and any integer M_i >= max_j x_ij (here ceil of the max),
    P~_ij = 2^(x_ij - M_i); P^ = P~ quantised in blocks of 32 consecutive keys of the row counted
    from the sequence's first key (masked entries are 0). A power-of-two factor commutes with the
    quantisation, so the result does not depend on which integer M_i is used;
  * out_i = sum_j P^_ij V^_j / sum_j P~_ij;  lse_i = ln sum_j exp(s_ij) over the visible keys.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from . import attention as A

E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest power of two (256) in E4M3
E4M3_EMIN = -6         # smallest normal exponent
E4M3_MBITS = 3
MX_BLOCK = 32


def e4m3_round(x):
    """Nearest E4M3 value of each element (ties to even), saturating at +-448; float64 in and out."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # quantum of the binade holding |x| (subnormals share the smallest normal binade's quantum)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, E4M3_EMIN)
    q = np.exp2(e - E4M3_MBITS)
    r = np.round(a / q) * q          # numpy rounds halves to even
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, x)


def mx_block_scale(amax):
    """E8M0 block scale 2^(floor(log2 amax) - 8) (2^-127 for an all-zero block)."""
    amax = np.asarray(amax, dtype=np.float64)
    e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - E4M3_EMAX
    return np.where(amax > 0, np.exp2(np.maximum(e, -127.0)), 2.0 ** -127)


def mx_quantize(x, axis: int = -1):
    """Dequantised MXFP8 value of ``x`` with blocks of 32 consecutive elements along ``axis`` (the
    axis length must be a multiple of 32; pad with zeros first)."""
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = x.shape[-1]
    if n % MX_BLOCK:
        raise ValueError("axis length must be a multiple of the block size")
    b = x.reshape(*x.shape[:-1], n // MX_BLOCK, MX_BLOCK)
    s = mx_block_scale(np.abs(b).max(axis=-1, keepdims=True))
    return np.moveaxis((e4m3_round(b / s) * s).reshape(x.shape), -1, axis)


def _quantize_seq_keys(v_seq):
    """[L, D] values of one sequence and head: blocks of 32 consecutive keys per feature."""
    L = v_seq.shape[0]
    pad = (-L) % MX_BLOCK
    vp = np.concatenate([v_seq, np.zeros((pad, v_seq.shape[1]))], axis=0) if pad else v_seq
    return mx_quantize(vp, axis=0)[:L]


def forward(q, k, v, q_off, kv_off, *, mask="none", bias_kind="none", bias=None, window=0, block=0,
            scale: Optional[float] = None, magnitude: bool = False):
    """MXFP8 softmax attention forward; returns ``(out [Tq, H, D], lse [H, Tq])``, and with
    ``magnitude`` also ``sum_j P^_ij |V^_jd| / sum_j P~_ij`` (the scale of each output element: a
    probability that rounds to the neighbouring E4M3 value, at most 2^-3 of itself away, moves
    the element by at most 2^-3 times this)."""
    q_off, kv_off = A._check(q, k, v, q_off, kv_off, mask, "softmax", bias_kind, bias, window, block)
    Tq, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    qh = mx_quantize(q, axis=-1)
    kh = mx_quantize(k, axis=-1)
    out = np.zeros((Tq, H, D))
    mag = np.zeros((Tq, H, D))
    lse = np.full((H, Tq), -np.inf)
    log2e = 1.0 / math.log(2.0)
    for b in range(len(q_off) - 1):
        qs, qe, ks, ke = q_off[b], q_off[b + 1], kv_off[b], kv_off[b + 1]
        lq, lkv = qe - qs, ke - ks
        if lq == 0 or lkv == 0:
            continue
        pad = (-lkv) % MX_BLOCK
        for h in range(H):
            K = kh[ks:ke, h]
            V = _quantize_seq_keys(v[ks:ke, h])
            bias_h = None if bias is None else np.asarray(bias, dtype=np.float64)[h]
            for i0, i1 in A._chunks(lq, lkv):
                S, vis, _ = A._scores(qh[qs + i0:qs + i1, h], K, i0, scale, mask, bias_kind, bias_h, window, block)
                x = np.where(vis, S * log2e, -np.inf)
                any_vis = vis.any(axis=1)
                M = np.ceil(np.where(any_vis, x.max(axis=1), 0.0))
                Pt = np.where(vis, np.exp2(x - M[:, None]), 0.0)
                Pq = mx_quantize(np.concatenate([Pt, np.zeros((Pt.shape[0], pad))], axis=1), axis=1)[:, :lkv]
                l = Pt.sum(axis=1)
                out[qs + i0:qs + i1, h] = np.where(any_vis[:, None], (Pq @ V) / np.where(any_vis, l, 1.0)[:, None], 0.0)
                if magnitude:
                    mag[qs + i0:qs + i1, h] = np.where(any_vis[:, None],
                                                       (Pq @ np.abs(V)) / np.where(any_vis, l, 1.0)[:, None], 0.0)
                with np.errstate(divide="ignore"):
                    lse[h, qs + i0:qs + i1] = np.where(any_vis, (M + np.log2(np.where(any_vis, l, 1.0))) / log2e,
                                                       -np.inf)
    return (out, lse, mag) if magnitude else (out, lse)
