"""Writes ``longtail_keycols.npz``: expected dK / dV of sampled keys of the longest sequences of the
long-tail workload, computed by the fp64 oracle (``oracle.attention.key_cols``) alone.

The long-tail workload (B = 512, Pareto(1.2) lengths from 128 clipped at 32,768, H = 8, D = 128, causal,
relative-position bucket bias) has two sequences of 32,768 tokens that carry half of its FLOPs. Their
whole dK / dV would take the oracle hours; each key's gradient needs only the statistics (lse_i,
Delta_i) of every query row that sees it plus its own score column, which ``key_cols`` computes
(the definition of the backward pass evaluated per key; aihot.vn GEM page, "Jagged Sequence Flash
Attention": efficient backward on jagged tensors). The first 512 sequences of ``longtail_1m`` are the
same sequences with the same values (one length stream and one value stream per workload id), so the
file serves both workloads.

Keys per (sequence, head): 16 in the first 128-key tile (whose dK/dV item walks all 512 query tiles),
16 in the last 128-key tile, 32 drawn uniformly; heads 0 and H - 1.

Run from the repository root: ``python tests/golden/make_longtail_keycols.py`` (four processes, a few
minutes on 8 cores). Imports only ``oracle`` and ``jfa_inputs``.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import jfa_inputs as ji  # noqa: E402
from oracle import attention as A  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "longtail_keycols.npz")


def sample_keys(L: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    first = np.concatenate([[0, 127], rng.choice(np.arange(1, 127), 14, replace=False)])
    last0 = (L - 1) // 128 * 128
    last = np.concatenate([[L - 1], rng.choice(np.arange(last0, L - 1), 15, replace=False)])
    used = set(first.tolist()) | set(last.tolist())
    rest = [j for j in rng.permutation(L).tolist() if j not in used][:32]
    return np.array(sorted(set(first.tolist()) | set(last.tolist()) | set(rest)), dtype=np.int64)


def _task(args):
    b, h, q, k, v, do, keys, kw = args
    from threadpoolctl import threadpool_limits
    t0 = time.perf_counter()
    with threadpool_limits(2):
        off = np.array([0, q.shape[0]], dtype=np.int32)
        dk, dv = A.key_cols(q, k, v, off, off, 0, h, keys, do, **kw)
    print(f"sequence {b} (L = {q.shape[0]}) head {h}: {len(keys)} keys in {time.perf_counter() - t0:.0f} s", flush=True)
    return b, h, dk.astype(np.float32), dv.astype(np.float32)


def main():
    import multiprocessing as mp
    name = "longtail"
    w = ji.WORKLOADS[name]
    x = ji.workload_inputs(name)
    lq, _ = ji.lengths(w)
    seqs = [int(b) for b in np.flatnonzero(lq == lq.max())]
    heads = [0, w.H - 1]
    f = A.bf16_bits_to_f64
    kw = dict(mask=w.mask, act=w.act, bias_kind=w.bias, bias=x.bias.astype(np.float64))
    rec = {"workload": np.array(name), "seqs": np.array(seqs), "heads": np.array(heads)}
    tasks = []
    for b in seqs:
        L = int(lq[b])
        qs, ks = int(x.q_off[b]), int(x.kv_off[b])
        q, k, v, do = (f(t[s:s + L]) for t, s in [(x.q, qs), (x.k, ks), (x.v, ks), (x.do, qs)])
        keys = sample_keys(L, b)
        rec[f"keys_{b}"] = keys
        tasks += [(b, h, q, k, v, do, keys, kw) for h in heads]
    del x
    # one (sequence, head) per process; the row statistics dominate (every score of the sequence)
    with mp.get_context("fork").Pool(len(tasks)) as pool:
        for b, h, dk, dv in pool.map(_task, tasks):
            rec[f"dk_{b}_{h}"] = dk
            rec[f"dv_{b}_{h}"] = dv
    np.savez_compressed(OUT, **rec)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
