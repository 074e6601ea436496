"""Helpers for the oracle's pins: padded dense attention through torch library routines.

Nothing here imports the oracle's arithmetic. The padded layout, the mask and the bias are built
independently (the bias bucket by enumerating interval boundaries), and softmax attention runs
through torch's own CPU attention kernels, so a mistake in the oracle cannot cancel out here.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F


def bucket_by_boundaries(d: np.ndarray) -> np.ndarray:
    """Bucket of |d| built by enumerating the start of every bucket interval.

    Buckets 0..15 start at 0..15; from 16 on, every octave [2^e, 2^(e+1)) is cut into four equal
    parts; bucket 63 absorbs everything from its start on.
    """
    starts = list(range(16))
    e = 4
    while len(starts) < 64:
        for part in range(4):
            starts.append(2 ** e + part * 2 ** (e - 2))
        e += 1
    starts = np.array(starts[:64], dtype=np.int64)
    a = np.abs(np.asarray(d, dtype=np.int64))
    return np.searchsorted(starts, a, side="right") - 1


def padded(x_f64: np.ndarray, off: np.ndarray, Lmax: int) -> torch.Tensor:
    """[T, H, D] jagged -> [B, H, Lmax, D] zero padded."""
    B = len(off) - 1
    T, H, D = x_f64.shape
    out = torch.zeros(B, H, Lmax, D, dtype=torch.float64)
    for b in range(B):
        s, e = int(off[b]), int(off[b + 1])
        out[b, :, : e - s] = torch.from_numpy(np.ascontiguousarray(x_f64[s:e].transpose(1, 0, 2)))
    return out


def unpad(x: torch.Tensor, off: np.ndarray) -> np.ndarray:
    """[B, H, Lmax, D] -> [T, H, D]."""
    parts = []
    for b in range(len(off) - 1):
        n = int(off[b + 1] - off[b])
        parts.append(x[b, :, :n].permute(1, 0, 2).detach().numpy())
    return np.concatenate(parts, axis=0) if parts else np.zeros((0,) + tuple(x.shape[1::2]))


def dense_bias_and_mask(q_off, kv_off, H, Lq, Lk, mask, bias_kind, bias, window=0, block=0):
    """Additive bias [B, H, Lq, Lk] and boolean visibility [B, 1, Lq, Lk] for the padded layout."""
    B = len(q_off) - 1
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    add = np.zeros((B, H, Lq, Lk))
    vis = np.zeros((B, 1, Lq, Lk), dtype=bool)
    for b in range(B):
        lq, lk = int(q_off[b + 1] - q_off[b]), int(kv_off[b + 1] - kv_off[b])
        v = (i < lq) & (j < lk)
        if mask == "causal":
            v &= j <= i
        if window:  # neighbours within the window: earlier ones only under the causal mask
            v &= (i - j < window) & ((mask == "causal") | (j - i < window))
        if block:  # same block of positions
            v &= (i // block) == (j // block)
        vis[b, 0] = v
        for h in range(H):
            if bias_kind == "scalar":
                add[b, h] = bias[h]
            elif bias_kind == "bucket":
                add[b, h] = np.asarray(bias[h], dtype=np.float64)[bucket_by_boundaries(i - j)]
    return torch.from_numpy(add), torch.from_numpy(vis)


def dense_softmax(q, k, v, q_off, kv_off, mask, bias_kind, bias, scale, want_grad=False, dout=None, window=0, block=0):
    """Softmax attention through torch's CPU attention kernels on a padded batch.

    Returns (out [Tq,H,D], lse [H,Tq]) and, with ``want_grad``, autograd gradients (dq, dk, dv,
    dbias) of <out, dout>. Padded query rows attend to key 0 only, so that no row is empty; they
    are dropped afterwards and receive zero output gradient.
    """
    H = q.shape[1]
    Lq = int(np.max(np.diff(q_off))) if len(q_off) > 1 else 0
    Lk = int(np.max(np.diff(kv_off))) if len(kv_off) > 1 else 0
    Q = padded(q, q_off, Lq).requires_grad_(want_grad)
    K = padded(k, kv_off, Lk).requires_grad_(want_grad)
    V = padded(v, kv_off, Lk).requires_grad_(want_grad)
    add, vis = dense_bias_and_mask(q_off, kv_off, H, Lq, Lk, mask, bias_kind, bias, window, block)
    bias_param = None
    if want_grad and bias_kind != "none":
        bias_param = torch.tensor(np.asarray(bias, dtype=np.float64), requires_grad=True)
        # rebuild the additive bias from the parameter so autograd reaches it
        idx = torch.from_numpy(bucket_by_boundaries(np.arange(Lq)[:, None] - np.arange(Lk)[None, :]))
        if bias_kind == "scalar":
            add = bias_param[None, :, None, None].expand(len(q_off) - 1, H, Lq, Lk)
        else:
            add = bias_param[:, idx][None].expand(len(q_off) - 1, H, Lq, Lk)
    row_pad = torch.zeros_like(vis)
    for b in range(len(q_off) - 1):
        lq = int(q_off[b + 1] - q_off[b])
        row_pad[b, 0, lq:, 0] = True
    allowed = vis | row_pad
    m = torch.where(allowed, add, torch.tensor(-math.inf, dtype=torch.float64))
    if want_grad:
        # the public entry point differentiates through the additive mask (bias gradient)
        out = F.scaled_dot_product_attention(Q, K, V, attn_mask=m, scale=scale)
        res = [unpad(out, q_off), None]
    else:
        out, lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
            Q, K, V, 0.0, False, attn_mask=m, scale=scale)
        res = [unpad(out, q_off), unpad(lse[..., None], q_off)[..., 0].T.copy()]
    if want_grad:
        dO = padded(dout, q_off, Lq)
        (out * dO).sum().backward()
        res += [unpad(Q.grad, q_off), unpad(K.grad, kv_off), unpad(V.grad, kv_off),
                None if bias_param is None else bias_param.grad.numpy()]
    return res


def dense_gdpa(q, k, v, q_off, kv_off, mask, act, bias_kind, bias, scale, want_grad=False, dout=None, window=0, block=0):
    """GDPA on a padded batch with torch's own activation routines (F.silu, F.gelu tanh)."""
    H = q.shape[1]
    Lq = int(np.max(np.diff(q_off)))
    Lk = int(np.max(np.diff(kv_off)))
    Q = padded(q, q_off, Lq).requires_grad_(want_grad)
    K = padded(k, kv_off, Lk).requires_grad_(want_grad)
    V = padded(v, kv_off, Lk).requires_grad_(want_grad)
    add, vis = dense_bias_and_mask(q_off, kv_off, H, Lq, Lk, mask, bias_kind, bias, window, block)
    bias_param = None
    if want_grad and bias_kind != "none":
        bias_param = torch.tensor(np.asarray(bias, dtype=np.float64), requires_grad=True)
        idx = torch.from_numpy(bucket_by_boundaries(np.arange(Lq)[:, None] - np.arange(Lk)[None, :]))
        if bias_kind == "scalar":
            add = bias_param[None, :, None, None].expand(len(q_off) - 1, H, Lq, Lk)
        else:
            add = bias_param[:, idx][None].expand(len(q_off) - 1, H, Lq, Lk)
    s = torch.matmul(Q, K.transpose(-1, -2).contiguous()) * scale + add
    a = F.silu(s) if act == "silu" else F.gelu(s, approximate="tanh")
    a = torch.where(vis, a, torch.zeros((), dtype=torch.float64))
    lk = torch.tensor(np.diff(kv_off).astype(np.float64))[:, None, None, None]
    out = torch.matmul(a, V) / lk
    res = [unpad(out, q_off)]
    if want_grad:
        dO = padded(dout, q_off, Lq)
        (out * dO).sum().backward()
        res += [unpad(Q.grad, q_off), unpad(K.grad, kv_off), unpad(V.grad, kv_off),
                None if bias_param is None else bias_param.grad.numpy()]
    return res
