"""Seeded synthetic inputs for jagged attention workloads.

This module draws sequence lengths and tensor values and nothing else: it holds none of the
attention arithmetic. Both the fp64 reference under ``oracle/`` and the GPU path read their
inputs from here, so the two see bit-identical operands.

The pages describe production recommendation traffic (user histories "from hundreds to tens of
thousands of tokens", short/asymmetric K/V, large batches; aihot.vn GEM page, sections "Jagged
Sequence Flash Attention" and "Generalized Dot-Product Attention"). No dataset is named, so the
workloads below are synthetic stand-ins with those length mixes.

Conventions (each one a reading where the pages are silent):
  * lengths: ``numpy.random.default_rng(0)`` (PCG64) for every workload; for the asymmetric
    workload the query lengths are drawn before the key/value lengths;
  * lognormal lengths: ``clip(rint(lognormal(ln median, 1.0)), lo, hi)``;
  * Pareto lengths: ``clip(floor((pareto(alpha) + 1) * x_min), x_min, hi)``;
  * tensor values: ``default_rng([workload_id, t])`` with t = 1 q, 2 k, 3 v, 4 dO, 5 bias;
    float32 standard-normal samples (times sigma for the bias) rounded to bfloat16 with
    round-to-nearest-even. The bias stays float32.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Stream ids for tensor values.
_T_Q, _T_K, _T_V, _T_DO, _T_BIAS = 1, 2, 3, 4, 5

MASKS = ("none", "causal")
ACTS = ("softmax", "silu", "gelu_tanh")
BIASES = ("none", "scalar", "bucket")
NUM_BUCKETS = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    """A named synthetic workload: length law, shape and attention mode."""
    name: str
    wid: int                      # stream id for tensor values
    B: int
    H: int
    D: int
    q_law: tuple                  # ("uniform", lo, hi_inclusive) | ("lognormal", median, lo, hi) | ("pareto", alpha, xmin, hi)
    kv_law: Optional[tuple]       # None: Lkv = Lq (self-attention)
    mask: str
    act: str
    bias: str
    bias_sigma: float = 0.0
    backward: bool = True
    description: str = ""
    window: int = 0               # sliding-window limit (0 = off)
    block: int = 0                # block-attention limit (0 = off)
    q_extra_law: Optional[tuple] = None  # target rows appended to each sequence's queries (fused self + target)
    shared_q: int = 0             # > 0: that many query rows shared by every sequence (PMA seeds)
    mxfp8: bool = False           # the forward pass in MXFP8


WORKLOADS = {
    w.name: w for w in [
        Workload("small_fwd", 1, 4, 2, 64, ("uniform", 16, 128), None, "none", "softmax", "none",
                 backward=False,
                 description="jagged softmax self-attention, forward only, B=4, L~U[16,128], H=2, D=64"),
        Workload("causal_bucket", 2, 64, 4, 128, ("lognormal", 512, 8, 4096), None, "causal", "softmax",
                 "bucket", 0.5,
                 description="jagged causal softmax self-attention, B=64, L~lognormal(512,1) in [8,4096], "
                             "H=4, D=128, 64-bucket relative bias ~N(0,0.5)"),
        Workload("target_attn", 3, 256, 8, 128, ("uniform", 1, 64), ("lognormal", 1024, 64, 16384), "none",
                 "softmax", "scalar", 0.1,
                 description="asymmetric target attention, B=256 users, Lq~U[1,64] candidates, "
                             "Lkv~lognormal(1024,1) in [64,16384] history, H=8, D=128, scalar bias ~N(0,0.1)"),
        Workload("gdpa_silu", 4, 128, 4, 128, ("lognormal", 800, 100, 8192), None, "causal", "silu", "none",
                 description="GDPA SiLU/Lkv, causal, B=128, L~lognormal(800,1) in [100,8192], H=4, D=128"),
        Workload("gdpa_gelu", 4, 128, 4, 128, ("lognormal", 800, 100, 8192), None, "causal", "gelu_tanh",
                 "none",
                 description="GDPA GELU-tanh/Lkv, causal, same lengths as gdpa_silu"),
        Workload("longtail", 5, 512, 8, 128, ("pareto", 1.2, 128, 32768), None, "causal", "softmax", "bucket",
                 0.5,
                 description="long-tail causal softmax, B=512, L=Pareto(1.2)*128 clipped to 32768, H=8, D=128, "
                             "64-bucket relative bias ~N(0,0.5)"),
        Workload("longtail_1m", 5, 1652, 8, 128, ("pareto", 1.2, 128, 32768), None, "causal", "softmax",
                 "bucket", 0.5,
                 description="as longtail, B=1652: the first batch of the same stream with >= 1M tokens"),
        # Sliding-window attention on the long-tail lengths: the pages apply it to long-sequence
        # self-attention and skip the tiles outside the window, without naming a window size;
        # 1024 keys (a few times the median length) is the stand-in.
        Workload("longtail_swa", 5, 512, 8, 128, ("pareto", 1.2, 128, 32768), None, "causal", "softmax",
                 "bucket", 0.5, window=1024,
                 description="as longtail with a causal sliding window of 1024 keys"),
        # Fused self + target attention (in-kernel broadcast inference co-designed with the model): each
        # user's history attends causally to itself and the user's candidates, appended after the
        # history, attend to the whole history, in one pass over one K/V copy per user. The pages give
        # no sizes; the history law is the causal workload's, the candidate count that of the
        # target-attention workload.
        Workload("self_target", 6, 256, 8, 128, ("lognormal", 512, 64, 4096), None, "causal", "softmax", "scalar",
                 0.1, q_extra_law=("uniform", 1, 64),
                 description="fused self + target: B=256 users, history~lognormal(512,1) in [64,4096] "
                             "(causal self-attention), then U[1,64] candidate rows that see the whole history; "
                             "H=8, D=128, scalar bias ~N(0,0.1)"),
        # The long-tail workload's forward pass in MXFP8 (the pages train attention in MXFP8).
        Workload("longtail_mxfp8", 5, 512, 8, 128, ("pareto", 1.2, 128, 32768), None, "causal", "softmax",
                 "bucket", 0.5, backward=False, mxfp8=True,
                 description="as longtail, forward only, in MXFP8 (E4M3 values, E8M0 scales per 32 elements)"),
        # Pooling by multihead attention: 32 learned seed queries shared by every sequence, attending
        # with a GDPA activation (the pages list PMA with self- and cross-attention under GDPA). The
        # pages give no sizes; the sequence law is the target-attention workload's history.
        Workload("pma_seeds", 7, 512, 8, 128, ("uniform", 32, 32), ("lognormal", 1024, 64, 16384), "none", "silu",
                 "none", shared_q=32,
                 description="PMA: 32 seed queries shared by B=512 sequences, Lkv~lognormal(1024,1) in "
                             "[64,16384], GDPA SiLU/Lkv, H=8, D=128"),
    ]
}


def _draw(law: tuple, n: int, rng: np.random.Generator) -> np.ndarray:
    kind = law[0]
    if kind == "uniform":
        _, lo, hi = law
        return rng.integers(lo, hi + 1, size=n).astype(np.int64)
    if kind == "lognormal":
        _, median, lo, hi = law
        x = rng.lognormal(np.log(median), 1.0, size=n)
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    if kind == "pareto":
        _, alpha, xmin, hi = law
        x = np.floor((rng.pareto(alpha, size=n) + 1.0) * xmin)
        return np.clip(x, xmin, hi).astype(np.int64)
    raise ValueError(f"unknown length law {law!r}")


def lengths(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    """Per-sequence (Lq, Lkv) as int64 arrays, drawn from ``default_rng(0)``."""
    rng = np.random.default_rng(0)
    if w.shared_q:
        return np.full(w.B, w.shared_q, dtype=np.int64), _draw(w.kv_law, w.B, rng)
    lq = _draw(w.q_law, w.B, rng)
    lkv = lq.copy() if w.kv_law is None else _draw(w.kv_law, w.B, rng)
    if w.q_extra_law is not None:  # queries = keys' rows followed by extra (target) rows
        lq = lq + _draw(w.q_extra_law, w.B, rng)
    return lq, lkv


def offsets(lens: np.ndarray) -> np.ndarray:
    """Exclusive prefix sum as int32 ``[B+1]`` with ``offsets[0] == 0``."""
    off = np.zeros(len(lens) + 1, dtype=np.int64)
    np.cumsum(np.asarray(lens, dtype=np.int64), out=off[1:])
    if off[-1] >= 2 ** 31:
        raise ValueError("total length exceeds int32")
    return off.astype(np.int32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_normal_bits(stream: tuple, n: int, chunk: int = 1 << 24) -> np.ndarray:
    """``n`` bf16 bit patterns of N(0,1) samples from ``default_rng(stream)``, drawn in chunks."""
    rng = np.random.default_rng(list(stream))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out


@dataclasses.dataclass
class Inputs:
    """One batch of jagged operands. Tensors are bf16 bit patterns (uint16) in ``[T, H, D]``."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: Optional[np.ndarray]
    bias: Optional[np.ndarray]    # float32 [H] (scalar) or [H, 64] (bucket); None when no bias
    q_off: np.ndarray             # int32 [B+1]
    kv_off: np.ndarray            # int32 [B+1]
    H: int
    D: int
    mask: str
    act: str
    bias_kind: str
    window: int = 0
    block: int = 0
    shared_q: bool = False        # q holds one set of Lq rows shared by every sequence

    @property
    def B(self) -> int:
        return len(self.q_off) - 1


def make_inputs(lq, lkv, H: int, D: int, *, wid: int, mask: str = "none", act: str = "softmax",
                bias_kind: str = "none", bias_sigma: float = 0.5, with_do: bool = True, window: int = 0,
                block: int = 0, shared_q: bool = False) -> Inputs:
    """Operands for arbitrary per-sequence lengths, from the value streams of id ``wid``.

    ``shared_q``: every Lq must be equal and ``q`` holds that many rows once, shared by all sequences
    (``dout`` stays per sequence)."""
    if mask not in MASKS or act not in ACTS or bias_kind not in BIASES:
        raise ValueError("bad mode")
    lq = np.asarray(lq, dtype=np.int64)
    lkv = np.asarray(lkv, dtype=np.int64)
    q_off, kv_off = offsets(lq), offsets(lkv)
    tq, tkv = int(q_off[-1]), int(kv_off[-1])
    if shared_q and len(set(lq.tolist())) > 1:
        raise ValueError("shared queries need equal Lq")
    nq = int(lq[0]) if shared_q and len(lq) else tq
    q = bf16_normal_bits((wid, _T_Q), nq * H * D).reshape(nq, H, D)
    k = bf16_normal_bits((wid, _T_K), tkv * H * D).reshape(tkv, H, D)
    v = bf16_normal_bits((wid, _T_V), tkv * H * D).reshape(tkv, H, D)
    do = bf16_normal_bits((wid, _T_DO), tq * H * D).reshape(tq, H, D) if with_do else None
    bias = None
    if bias_kind != "none":
        shape = (H,) if bias_kind == "scalar" else (H, NUM_BUCKETS)
        rng = np.random.default_rng([wid, _T_BIAS])
        bias = (rng.standard_normal(int(np.prod(shape)), dtype=np.float32) * np.float32(bias_sigma)).reshape(shape)
    return Inputs(q, k, v, do, bias, q_off, kv_off, H, D, mask, act, bias_kind, int(window), int(block),
                  bool(shared_q))


def workload_inputs(name: str, with_do: Optional[bool] = None) -> Inputs:
    """Full-size operands of a named workload."""
    w = WORKLOADS[name]
    lq, lkv = lengths(w)
    if with_do is None:
        with_do = w.backward
    return make_inputs(lq, lkv, w.H, w.D, wid=w.wid, mask=w.mask, act=w.act, bias_kind=w.bias,
                       bias_sigma=w.bias_sigma, with_do=with_do, window=w.window, block=w.block,
                       shared_q=w.shared_q > 0)
