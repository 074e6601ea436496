"""Pins of the seeded input generator (CPU)."""
import numpy as np
import pytest
import torch

import jfa_inputs as ji

# integers of the seed-0 draws (numpy 2.2 PCG64), per workload: (tokens q, tokens kv, max length)
EXPECT = {
    "small_fwd": (318, 318, 112),
    "causal_bucket": (52528, 52528, 3636),
    "target_attn": (8668, 409834, None),
    "gdpa_silu": (166288, 166288, 5925),
    "longtail": (333877, 333877, 32768),
    "longtail_1m": (1000301, 1000301, 32768),
}


@pytest.mark.parametrize("name", list(EXPECT))
def test_length_draws(name):
    lq, lkv = ji.lengths(ji.WORKLOADS[name])
    tq, tk, mx = EXPECT[name]
    assert int(lq.sum()) == tq and int(lkv.sum()) == tk
    if mx is not None:
        assert int(lq.max()) == mx


def test_small_workload_lengths():
    lq, lkv = ji.lengths(ji.WORKLOADS["small_fwd"])
    assert lq.tolist() == [112, 87, 73, 46] and lkv.tolist() == lq.tolist()


def test_length_laws_respect_bounds():
    lq, lkv = ji.lengths(ji.WORKLOADS["target_attn"])
    assert lq.min() >= 1 and lq.max() <= 64 and lkv.min() >= 64 and lkv.max() <= 16384
    lq, _ = ji.lengths(ji.WORKLOADS["longtail"])
    assert lq.min() >= 128 and (lq == 32768).sum() == 2 and np.median(lq) == 247
    # the first B of the 1M-token stream is the B=512 batch
    l1m, _ = ji.lengths(ji.WORKLOADS["longtail_1m"])
    np.testing.assert_array_equal(l1m[:512], lq)
    assert l1m[:1651].sum() < 1_000_000 <= l1m.sum()


def test_offsets():
    off = ji.offsets(np.array([3, 0, 5]))
    assert off.dtype == np.int32 and off.tolist() == [0, 3, 3, 8]


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(100000, dtype=np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 3.0e38], dtype=np.float32)])
    x = x.astype(np.float32)
    ours = ji.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_value_streams_are_reproducible_and_chunk_independent():
    a = ji.bf16_normal_bits((2, 1), 100_000)
    b = ji.bf16_normal_bits((2, 1), 100_000, chunk=777)
    np.testing.assert_array_equal(a, b)
    c = ji.bf16_normal_bits((2, 2), 100_000)
    assert not np.array_equal(a, c)
    x = ji.make_inputs([3, 4], [5, 6], 2, 8, wid=9, bias_kind="bucket", bias_sigma=0.5)
    assert x.q.shape == (7, 2, 8) and x.k.shape == (11, 2, 8) and x.bias.shape == (2, 64)
    assert x.bias.dtype == np.float32
