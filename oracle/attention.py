"""fp64 reference of jagged attention, forward and backward (test infrastructure only).

Operands are packed jagged tensors: ``q``, ``dout`` are ``[Tq, H, D]`` and ``k``, ``v`` are
``[Tkv, H, D]`` with sequence ``b`` in rows ``off[b]:off[b+1]`` (values + offsets, vibekk.com GEM
page, FAQ entry on jagged tensors). Nothing is padded: each (sequence, head) is handled on its
own slice. Query rows are processed in chunks so that the longest sequence fits in memory; the
chunking changes no arithmetic beyond the order of independent rows.

For one sequence b and head h (i < Lq_b, j < Lkv_b):

  s_ij   = scale * <Q_i, K_j> + beta_h(i, j)        beta: 0 | c_h | T[h, bucket(i - j)]
  vis_ij = base_ij and window_ij and block_ij
    base:   (mask == none) or (j <= i)
    window: W == 0, or i - j < W (and, without the causal mask, also j - i < W)
    block:  B == 0, or floor(i / B) == floor(j / B)

The window and block limits follow the pages' long-sequence masks: sliding-window attention
limits each token to neighbouring events and its kernel skips the tiles outside the window
(aihot.vn GEM page, "BlockAttention"), and BlockAttention cuts a long sequence into independent
fixed blocks (vibekk.com GEM page, section on moving from padding to jagged kernels;
kerneldigest.dev page, "Arquitectura del Sistema"). The pages fix neither the window's side nor the block's interior;
here a window under the causal mask looks back only, and a block keeps the base mask inside it.
GDPA keeps its 1 / Lkv_b normalisation under both.

softmax (FlashAttention's result on jagged tensors; aihot.vn GEM page, "Jagged Sequence Flash
Attention"; kerneldigest.dev page, "Fundamentos Teóricos"):

  P_ij = exp(s_ij - m_i) / l_i on visible pairs,  m_i = max_vis s_ij,  l_i = sum_vis exp(s_ij - m_i)
  O_i  = sum_j P_ij V_j,   lse_i = m_i + ln l_i;    a row with nothing visible gives O_i = 0, lse_i = -inf

GDPA (two matrix products with a pointwise activation in place of softmax; aihot.vn GEM page,
"Generalized Dot-Product Attention (GDPA)"), normalised by the sequence's key count:

  O_i = (1 / Lkv_b) sum_vis act(s_ij) V_j,   act = SiLU or GELU (tanh form)

Masked pairs contribute exactly nothing in both modes: the pages describe masking "by
subtraction" (kerneldigest.dev page, "Arquitectura del Sistema") — a device mechanism, read here
as exclusion.

Under the causal mask a sequence may have more queries than keys (Lq_b >= Lkv_b): the fused self +
target pass of in-kernel broadcast inference (itsolotime.com IKBO page, table of contents section
3.3, "Self + Target attention fused through model co-design"). Rows i < Lkv_b are the user's history
attending causally to itself; rows i >= Lkv_b are target (candidate) rows, and j <= i then holds for
every key, so each target sees the whole history and nothing else — the same result as a separate
cross-attention of the targets on the history (positions, and hence a relative-position bias, still
count from the sequence start).

The backward pass is the gradient of <O, dO> (plus nothing from lse) with respect to q, k, v and
the bias parameters, written out:

  softmax: dP = dO V^T, Delta_i = sum_j P_ij dP_ij, dS = P (dP - Delta)
  GDPA:    dP = dO V^T / Lkv_b, dS = dP act'(s) on visible pairs
  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO (softmax) | act(s)^T dO / Lkv_b (GDPA)
  dc_h = sum dS,    dT[h, u] = sum of dS over pairs with bucket(i - j) = u
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .bucket import NUM_BUCKETS, bucket

_SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
_GELU_C = 0.044715
_ROW_CHUNK_ELEMS = 1 << 23      # bound on rows * Lkv per chunk (64 MiB of fp64 scores)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def silu(x):
    """SiLU(x) = x / (1 + exp(-x))."""
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def silu_grad(x):
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-x))
    return sig * (1.0 + x * (1.0 - sig))


def gelu_tanh(x):
    """GELU, tanh form: x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    return 0.5 * x * (1.0 + np.tanh(_SQRT_2_OVER_PI * (x + _GELU_C * x ** 3)))


def gelu_tanh_grad(x):
    t = np.tanh(_SQRT_2_OVER_PI * (x + _GELU_C * x ** 3))
    du = _SQRT_2_OVER_PI * (1.0 + 3.0 * _GELU_C * x ** 2)
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * du


_ACTS = {"silu": (silu, silu_grad), "gelu_tanh": (gelu_tanh, gelu_tanh_grad)}


def _check(q, k, v, q_off, kv_off, mask, act, bias_kind, bias, window=0, block=0):
    q_off = np.asarray(q_off, dtype=np.int64)
    kv_off = np.asarray(kv_off, dtype=np.int64)
    if q_off.ndim != 1 or q_off.shape != kv_off.shape or len(q_off) < 2:
        raise ValueError("offsets must be [B+1]")
    if q_off[0] != 0 or kv_off[0] != 0 or np.any(np.diff(q_off) < 0) or np.any(np.diff(kv_off) < 0):
        raise ValueError("offsets must start at 0 and be non-decreasing")
    if q.shape[0] != q_off[-1] or k.shape[0] != kv_off[-1] or v.shape != k.shape:
        raise ValueError("tensor rows do not match offsets")
    if mask not in ("none", "causal") or act not in ("softmax", "silu", "gelu_tanh"):
        raise ValueError("bad mode")
    if int(window) != window or window < 0 or int(block) != block or block < 0:
        raise ValueError("window and block must be integers >= 0")
    H = q.shape[1]
    if bias_kind == "scalar":
        assert bias is not None and np.shape(bias) == (H,)
    elif bias_kind == "bucket":
        assert bias is not None and np.shape(bias) == (H, NUM_BUCKETS)
    elif bias_kind != "none":
        raise ValueError("bad bias kind")
    return q_off, kv_off


def visible(i, j, mask, window=0, block=0):
    """Visibility of query position i and key position j (numpy broadcasting)."""
    vis = (j <= i) if mask == "causal" else np.ones(np.broadcast(i, j).shape, dtype=bool)
    if window:
        vis = vis & (i - j < window)
        if mask != "causal":
            vis = vis & (j - i < window)
    if block:
        vis = vis & (i // block == j // block)
    return vis


def _scores(Qc, K, i0, scale, mask, bias_kind, bias_h, window=0, block=0):
    """Scores and visibility of query rows i0.. of one (sequence, head) against all its keys."""
    rows, lkv = Qc.shape[0], K.shape[0]
    S = scale * (Qc @ K.T)
    i = i0 + np.arange(rows)[:, None]
    j = np.arange(lkv)[None, :]
    if bias_kind == "scalar":
        S = S + bias_h
    elif bias_kind == "bucket":
        S = S + bias_h[bucket(i - j)]
    vis = visible(i, j, mask, window, block) & np.ones((rows, lkv), dtype=bool)
    return S, vis, i - j


def _softmax_rows(S, vis):
    """Normalised probabilities and log-sum-exp of each row over its visible entries."""
    any_vis = vis.any(axis=1)
    m = np.where(vis, S, -np.inf).max(axis=1, initial=-np.inf)
    m_safe = np.where(any_vis, m, 0.0)
    E = np.where(vis, np.exp(S - m_safe[:, None]), 0.0)
    l = E.sum(axis=1)
    P = np.where(any_vis[:, None], E / np.where(any_vis, l, 1.0)[:, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(any_vis, m + np.log(np.where(any_vis, l, 1.0)), -np.inf)
    return P, lse


def _chunks(lq, lkv):
    step = max(1, min(1024, _ROW_CHUNK_ELEMS // max(1, lkv)))
    for i0 in range(0, lq, step):
        yield i0, min(lq, i0 + step)


def _select(n, subset):
    return range(n) if subset is None else subset


def forward(q, k, v, q_off, kv_off, *, mask="none", act="softmax", bias_kind="none", bias=None, window=0, block=0,
            scale: Optional[float] = None, seqs: Optional[Sequence[int]] = None,
            heads: Optional[Sequence[int]] = None):
    """Attention output ``[Tq, H, D]`` and, for softmax, ``lse [H, Tq]`` (natural log).

    ``q``, ``k``, ``v`` are float64 (use :func:`bf16_bits_to_f64` for bf16 operands). ``seqs`` /
    ``heads`` restrict the work to a subset; entries outside it are left NaN.
    """
    q_off, kv_off = _check(q, k, v, q_off, kv_off, mask, act, bias_kind, bias, window, block)
    Tq, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.full((Tq, H, D), np.nan)
    lse = np.full((H, Tq), np.nan) if act == "softmax" else None
    for b in _select(len(q_off) - 1, seqs):
        qs, qe, ks, ke = q_off[b], q_off[b + 1], kv_off[b], kv_off[b + 1]
        lq, lkv = qe - qs, ke - ks
        for h in _select(H, heads):
            K, V = k[ks:ke, h], v[ks:ke, h]
            bias_h = None if bias is None else np.asarray(bias, dtype=np.float64)[h]
            for i0, i1 in _chunks(lq, lkv):
                S, vis, _ = _scores(q[qs + i0:qs + i1, h], K, i0, scale, mask, bias_kind, bias_h, window, block)
                if act == "softmax":
                    P, lse_c = _softmax_rows(S, vis)
                    out[qs + i0:qs + i1, h] = P @ V
                    lse[h, qs + i0:qs + i1] = lse_c
                else:
                    f, _ = _ACTS[act]
                    A = np.where(vis, f(S), 0.0)
                    out[qs + i0:qs + i1, h] = (A @ V) / lkv if lkv > 0 else 0.0
    return out, lse


def backward(q, k, v, q_off, kv_off, dout, *, mask="none", act="softmax", bias_kind="none", bias=None, window=0, block=0,
             scale: Optional[float] = None, seqs: Optional[Sequence[int]] = None,
             heads: Optional[Sequence[int]] = None):
    """Gradients ``(dq, dk, dv, dbias)`` of ``<forward(...).out, dout>``.

    ``dbias`` has the bias shape (``[H]`` or ``[H, 64]``) or is None without a bias; when
    ``seqs`` / ``heads`` select a subset, ``dbias`` sums over that subset only.
    """
    q_off, kv_off = _check(q, k, v, q_off, kv_off, mask, act, bias_kind, bias, window, block)
    Tq, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    dbias = None if bias is None else np.zeros(np.shape(bias))
    for b in _select(len(q_off) - 1, seqs):
        qs, qe, ks, ke = q_off[b], q_off[b + 1], kv_off[b], kv_off[b + 1]
        lq, lkv = qe - qs, ke - ks
        for h in _select(H, heads):
            K, V = k[ks:ke, h], v[ks:ke, h]
            bias_h = None if bias is None else np.asarray(bias, dtype=np.float64)[h]
            dK = np.zeros((lkv, D))
            dV = np.zeros((lkv, D))
            for i0, i1 in _chunks(lq, lkv):
                Qc = q[qs + i0:qs + i1, h]
                dOc = dout[qs + i0:qs + i1, h]
                S, vis, rel = _scores(Qc, K, i0, scale, mask, bias_kind, bias_h, window, block)
                if act == "softmax":
                    P, _ = _softmax_rows(S, vis)
                    dP = dOc @ V.T
                    delta = (P * dP).sum(axis=1)
                    dS = P * (dP - delta[:, None])
                    dV += P.T @ dOc
                else:
                    f, fprime = _ACTS[act]
                    inv_l = 1.0 / lkv if lkv > 0 else 0.0
                    A = np.where(vis, f(S), 0.0)
                    dP = (dOc @ V.T) * inv_l
                    dS = np.where(vis, dP * fprime(S), 0.0)
                    dV += (A.T @ dOc) * inv_l
                dq[qs + i0:qs + i1, h] = scale * (dS @ K)
                dK += scale * (dS.T @ Qc)
                if bias_kind == "scalar":
                    dbias[h] += dS.sum()
                elif bias_kind == "bucket":
                    dbias[h] += np.bincount(bucket(rel[vis]), weights=dS[vis], minlength=NUM_BUCKETS)
            dk[ks:ke, h] = dK
            dv[ks:ke, h] = dV
    return dq, dk, dv, dbias


def gdpa_magnitude(q, k, v, q_off, kv_off, *, mask="none", act="silu", bias_kind="none", bias=None, window=0, block=0,
                   scale: Optional[float] = None, seqs=None, heads=None):
    """(1 / Lkv_b) sum_vis |act(s_ij)| |V_jd|: the scale of each GDPA output element.

    Rounding act(s) to a bfloat16 matrix operand changes output element (i, d) by at most the unit
    roundoff 2^-8 times this magnitude; GPU tolerances for GDPA use it.
    """
    if act == "softmax":
        raise ValueError("GDPA only")
    q_off, kv_off = _check(q, k, v, q_off, kv_off, mask, act, bias_kind, bias, window, block)
    Tq, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.full((Tq, H, D), np.nan)
    f, _ = _ACTS[act]
    for b in _select(len(q_off) - 1, seqs):
        qs, qe, ks, ke = q_off[b], q_off[b + 1], kv_off[b], kv_off[b + 1]
        lq, lkv = qe - qs, ke - ks
        for h in _select(H, heads):
            K, V = k[ks:ke, h], np.abs(v[ks:ke, h])
            bias_h = None if bias is None else np.asarray(bias, dtype=np.float64)[h]
            for i0, i1 in _chunks(lq, lkv):
                S, vis, _ = _scores(q[qs + i0:qs + i1, h], K, i0, scale, mask, bias_kind, bias_h, window, block)
                Aa = np.where(vis, np.abs(f(S)), 0.0)
                out[qs + i0:qs + i1, h] = (Aa @ V) / lkv if lkv > 0 else 0.0
    return out



def rows(q, k, v, q_off, kv_off, b, h, rows_, dout=None, *, mask="none", act="softmax", bias_kind="none", bias=None,
         window=0, block=0, scale: Optional[float] = None):
    """Output, log-sum-exp (softmax) and, given ``dout``, dQ of selected query rows of one sequence and
    head, each from its own score row against all the sequence's keys.

    The same definition as :func:`forward` and :func:`backward`, evaluated one query row at a time, so
    that single outputs of very long sequences can be checked without the whole score matrix. Returns
    ``(out [n, D], lse [n] or None, dq [n, D] or None)``.
    """
    q_off, kv_off = _check(q, k, v, q_off, kv_off, mask, act, bias_kind, bias, window, block)
    D = q.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    qs, ks, ke = q_off[b], kv_off[b], kv_off[b + 1]
    lkv = ke - ks
    K, V = k[ks:ke, h], v[ks:ke, h]
    bias_h = None if bias is None else np.asarray(bias, dtype=np.float64)[h]
    n = len(rows_)
    out, lse = np.zeros((n, D)), (np.zeros(n) if act == "softmax" else None)
    dq = None if dout is None else np.zeros((n, D))
    for r, i in enumerate(rows_):
        S, vis, _ = _scores(q[qs + i:qs + i + 1, h], K, i, scale, mask, bias_kind, bias_h, window, block)
        if act == "softmax":
            P, l = _softmax_rows(S, vis)
            out[r], lse[r] = (P @ V)[0], l[0]
            if dout is not None:
                dP = dout[qs + i:qs + i + 1, h] @ V.T
                dS = P * (dP - (P * dP).sum())
                dq[r] = scale * (dS @ K)[0]
        else:
            f, fprime = _ACTS[act]
            inv_l = 1.0 / lkv if lkv > 0 else 0.0
            out[r] = (np.where(vis, f(S), 0.0) @ V)[0] * inv_l
            if dout is not None:
                dS = np.where(vis, (dout[qs + i:qs + i + 1, h] @ V.T) * inv_l * fprime(S), 0.0)
                dq[r] = scale * (dS @ K)[0]
    return out, lse, dq


def key_cols(q, k, v, q_off, kv_off, b, h, keys, dout, *, mask="none", act="softmax", bias_kind="none", bias=None,
             window=0, block=0, scale: Optional[float] = None):
    """dK and dV of selected keys of one sequence and head, each from its own column of scores.

    The same definition as :func:`backward`, evaluated per key j: with the row statistics of every
    query i that sees j (softmax: lse_i and Delta_i = sum_j' P_ij' dP_ij' over the whole row),

      softmax: P_ij = exp(s_ij - lse_i), dS_ij = P_ij (<dO_i, V_j> - Delta_i)
      GDPA:    P_ij = act(s_ij) / Lkv,   dS_ij = <dO_i, V_j> act'(s_ij) / Lkv
      dK_j = scale sum_i dS_ij Q_i,      dV_j = sum_i P_ij dO_i

    so that single keys of very long sequences can be checked without all of dK. The row statistics
    come from the full score rows, processed in chunks of query rows. Returns ``(dk [n, D], dv [n, D])``.
    """
    q_off, kv_off = _check(q, k, v, q_off, kv_off, mask, act, bias_kind, bias, window, block)
    D = q.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    qs, qe, ks, ke = q_off[b], q_off[b + 1], kv_off[b], kv_off[b + 1]
    lq, lkv = qe - qs, ke - ks
    K, V = k[ks:ke, h], v[ks:ke, h]
    keys = np.asarray(keys, dtype=np.int64)
    bias_h = None if bias is None else np.asarray(bias, dtype=np.float64)[h]
    dk = np.zeros((len(keys), D))
    dv = np.zeros((len(keys), D))
    for i0, i1 in _chunks(lq, lkv):
        Qc = q[qs + i0:qs + i1, h]
        dOc = dout[qs + i0:qs + i1, h]
        # full rows: the statistics each query row contributes to every key column
        S, vis, _ = _scores(Qc, K, i0, scale, mask, bias_kind, bias_h, window, block)
        if act == "softmax":
            P, lse = _softmax_rows(S, vis)
            delta = (P * (dOc @ V.T)).sum(axis=1)
        del S, vis
        # the selected key columns, at their positions j in the sequence
        Sk = scale * (Qc @ K[keys].T)
        i = i0 + np.arange(i1 - i0)[:, None]
        j = keys[None, :]
        if bias_kind == "scalar":
            Sk = Sk + bias_h
        elif bias_kind == "bucket":
            Sk = Sk + bias_h[bucket(i - j)]
        visk = visible(i, j, mask, window, block) & (j < lkv)
        dPk = dOc @ V[keys].T
        if act == "softmax":
            with np.errstate(invalid="ignore"):
                Pk = np.where(visk & np.isfinite(lse)[:, None], np.exp(Sk - np.where(np.isfinite(lse), lse, 0.0)[:, None]), 0.0)
            dSk = Pk * (dPk - delta[:, None])
        else:
            f, fprime = _ACTS[act]
            inv_l = 1.0 / lkv if lkv > 0 else 0.0
            Pk = np.where(visk, f(Sk), 0.0) * inv_l
            dSk = np.where(visk, dPk * inv_l * fprime(Sk), 0.0)
        dk += scale * (dSk.T @ Qc)
        dv += Pk.T @ dOc
    return dk, dv


def replicate_shared_q(q_shared, num_seqs: int):
    """Query rows of every sequence when one set of ``Ls`` query rows is shared by all of them.

    Pooling by multihead attention (PMA), which the pages list beside self- and cross-attention as the
    same two-product structure (aihot.vn GEM page, "Generalized Dot-Product Attention (GDPA)"), attends
    from one learned set of seed queries to each sequence's keys: sequence b's queries are the seeds
    themselves. Returns the explicit copy ``[B * Ls, H, D]`` and its offsets ``b * Ls``; the device
    reads the shared rows without making it.
    """
    q_shared = np.asarray(q_shared)
    Ls = q_shared.shape[0]
    return np.tile(q_shared, (num_seqs, 1, 1)), np.arange(num_seqs + 1, dtype=np.int64) * Ls


def forward_shared_q(q_shared, k, v, kv_off, **kw):
    """:func:`forward` with the query rows shared by every sequence (see :func:`replicate_shared_q`)."""
    B = len(kv_off) - 1
    q_rep, q_off = replicate_shared_q(q_shared, B)
    return forward(q_rep, k, v, q_off, kv_off, **kw)


def backward_shared_q(q_shared, k, v, kv_off, dout, **kw):
    """:func:`backward` with shared query rows: the gradient of a query row used by every sequence is
    the sum of its gradients in each sequence (the chain rule over its B uses). Returns
    ``(dq [Ls, H, D], dk, dv, dbias)``."""
    B = len(kv_off) - 1
    q_rep, q_off = replicate_shared_q(q_shared, B)
    dq, dk, dv, db = backward(q_rep, k, v, q_off, kv_off, dout, **kw)
    Ls = np.asarray(q_shared).shape[0]
    return dq.reshape(B, Ls, *dq.shape[1:]).sum(axis=0), dk, dv, db
